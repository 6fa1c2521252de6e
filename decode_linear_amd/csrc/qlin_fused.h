// The fused decode-time linear for gfx950 (CDNA4, wave64), shared by the four format
// instantiations (qlin_fused_{q4,q8,f16,bf16}.hip).
//
// What it computes ([p1] maya-mac src/maya_mac/mlx_kernels.py, `_linear_kernel`):
//   y[t, n] = epi( LN?(x_t) . W_n )   with   W[n, k] = q[n, k] * s[n, k/64] + b[n, k/64]
// LayerNorm is folded into the weight stream with the identity stated in that kernel's
// docstring, LN(x).w = rstd * (sum (x - x0) g w - (mean - x0) sum g w) + sum b w, using the
// single-pass statistics of x shifted by x0 = x[t, 0].  The per-group dequantization is
// factored out of the inner product ([p3] mlx-bun 0.0.10 -> 0.0.12, fused-decode-kernel.ts,
// the "qdot pattern"):  sum_k (s q_k + b) a_k = s * sum_k q_k a_k + b * sum_k a_k.
//
// How it maps onto CDNA4:
//   * One workgroup = 8 waves, about one workgroup per CU; workgroup b visits output tiles
//     b, b + grid, ...  Wave w owns a fixed slice of K for the whole launch.
//   * Staging (once per launch, or once per K chunk when K is long): the workgroup reads
//     the activation rows (x, gamma, beta) with coalesced 16-byte loads, one source row per
//     wave, and writes the MFMA operand rows into LDS: per-row power-of-two scale into the
//     fp16 range, split into 1-3 16-bit terms so the operand carries >= 22 significant bits,
//     plus per-group sums for the bias product and the shifted LayerNorm sums (all row
//     reductions are fixed-order wave butterflies).  Each wave then loads its slice's
//     fragments into VGPRs; the LDS is reused for the cross-wave merge.
//   * Weight stream: lane (c, i) of a wave (c = lane/16, i = lane%16) reads 16 bytes of
//     weight row i per 64-byte step (a dwordx4); 64 lanes cover 16 rows x 64 contiguous
//     bytes per instruction.  The next tile's loads are issued before the current tile is
//     computed.
//   * Contraction: v_mfma_f32_16x16x32_{f16,bf16}.  B = 16 weight rows x 32 k of exactly
//     converted codes (integers 0..255 are exact in fp16): 8-bit codes become fp16 with a
//     byte permute under the exponent of 1024 and a packed subtract; 4-bit nibbles the same
//     way with masks (odd nibbles sit 4 bits higher and are rescaled by an exact packed FMA).
//     A = up to 16 operand rows x 32 k.  LayerNorm adds the rows gamma and beta, whose
//     products give sum g w and sum b w for the fold.
//   * Per group of 64 codes the MFMA output is a fresh partial P and acc += s * P; the bias
//     term sum_g b * (sum of the group's operands) is one more MFMA per tile (group sums as
//     an fp16 hi/lo operand against the exact fp16 biases).
//   * 4-bit rows hold two groups per 64-byte step; after the load, v_permlane32_swap
//     exchanges half-registers between the lane halves so that every MFMA sees one group.
//   * No atomics: partial sums merge in a fixed order (waves, then terms), so results are
//     bitwise reproducible.
#pragma once

#include "qlin_internal.h"

namespace qlin {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// Per weight format: MFMAs per 64-byte step and quantization groups per step.
template <int BITS> struct Fmt;
template <> struct Fmt<4> { static constexpr int kMfma = 4, kGroups = 2, kStepK = 128; };
template <> struct Fmt<8> { static constexpr int kMfma = 2, kGroups = 1, kStepK = 64; };
template <> struct Fmt<16> { static constexpr int kMfma = 1, kGroups = 0, kStepK = 32; };

// VGPRs allowed for the register-resident activation fragments.
constexpr int kFragBudget = 80;
__host__ __device__ constexpr int max_steps_for(int mfma, int mt) {
  return (kFragBudget / (4 * mfma * mt)) < 1 ? 1 : ((kFragBudget / (4 * mfma * mt)) > 8 ? 8 : (kFragBudget / (4 * mfma * mt)));
}

// First k (within a step) of the 8 consecutive k that lane group c feeds to MFMA q.
// 4-bit: the 16 loaded bytes of lane group c hold codes 32c..32c+31 of the step; after
// swapping the upper half of dword 0 with the lower half of dword 1 (and dwords 2/3),
// dwords 0 and 2 hold group 0 and dwords 1 and 3 group 1.  MFMA order: dword 0, 2, 1, 3.
template <int BITS> __device__ __forceinline__ int frag_base(int q, int c) {
  if constexpr (BITS == 16) return 8 * c;
  else if constexpr (BITS == 8) return 16 * c + 8 * q;
  else return (c & 1) * 32 + (c >> 1) * 8 + (q & 1) * 16 + (q >> 1) * 64;
}
// Position of operand slot j among those 8 k (4-bit conversion emits nibbles 0,4,1,5,2,6,3,7).
template <int BITS> __device__ __forceinline__ int slot_k(int j) {
  if constexpr (BITS == 4) return (j & 1) * 4 + (j >> 1);
  else return j;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float elem_to_float(uint32_t h, int dtype) {
  return dtype == 1 ? half_bits_to_float(h) : __builtin_bit_cast(float, h << 16);
}

// 8 consecutive 16-bit elements at base[idx..idx+7] (idx % 8 == 0, base 16-byte aligned).
__device__ __forceinline__ void load8(const void* base, int dtype, long idx, float v[8]) {
  const u4_t raw = *reinterpret_cast<const u4_t*>(reinterpret_cast<const uint16_t*>(base) + idx);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = elem_to_float((raw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu, dtype);
}

// ---- code conversion to fp16 operand pairs ------------------------------------------
// Byte pair of an 8-bit word -> two fp16 integers.  v_perm puts code bytes under the
// exponent byte 0x64 (fp16 1024 has unit spacing), then 1024 is subtracted exactly.
__device__ __forceinline__ uint32_t bytes_to_h2(uint32_t d, uint32_t sel) {
  const uint32_t h = __builtin_amdgcn_perm(0x64646464u, d, sel);
  const h2_t v = __builtin_bit_cast(h2_t, h) - (h2_t){(_Float16)1024.0f, (_Float16)1024.0f};
  return __builtin_bit_cast(uint32_t, v);
}
// Nibbles 0 and 4 of d (bits 0-3 and 16-19) -> fp16 integers.
// (a & mask) | magic as one v_and_or_b32.  gfx9 VOP3 cannot encode 32-bit literals, so
// without this the compiler emits a separate v_and and v_or; the mask goes in an SGPR and
// the magic constant in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}
__device__ __forceinline__ uint32_t nib_lo_to_h2(uint32_t d) {
  const uint32_t h = and_or(d, 0x000F000Fu, 0x64006400u);
  const h2_t v = __builtin_bit_cast(h2_t, h) - (h2_t){(_Float16)1024.0f, (_Float16)1024.0f};
  return __builtin_bit_cast(uint32_t, v);
}
// Nibbles 1 and 5 (bits 4-7 and 20-23): 1024 + 16 n, scaled back exactly: (1024+16n)/16 - 64.
__device__ __forceinline__ uint32_t nib_hi_to_h2(uint32_t d) {
  const uint32_t h = and_or(d, 0x00F000F0u, 0x64006400u);
  const h2_t v = __builtin_elementwise_fma(__builtin_bit_cast(h2_t, h), (h2_t){(_Float16)0.0625f, (_Float16)0.0625f},
                                           (h2_t){(_Float16)-64.0f, (_Float16)-64.0f});
  return __builtin_bit_cast(uint32_t, v);
}

template <int BITS>
__device__ __forceinline__ u4_t convert_codes(const u4_t d, int q) {
  u4_t b;
  if constexpr (BITS == 8) {
    const uint32_t da = d[2 * q], db = d[2 * q + 1];
    b[0] = bytes_to_h2(da, 0x04010400u);
    b[1] = bytes_to_h2(da, 0x04030402u);
    b[2] = bytes_to_h2(db, 0x04010400u);
    b[3] = bytes_to_h2(db, 0x04030402u);
  } else if constexpr (BITS == 4) {
    const uint32_t r = d[(q & 1) * 2 + (q >> 1)];
    b[0] = nib_lo_to_h2(r);
    b[1] = nib_hi_to_h2(r);
    b[2] = nib_lo_to_h2(r >> 8);
    b[3] = nib_hi_to_h2(r >> 8);
  } else {
    b = d;
  }
  return b;
}

template <bool BF16OP>
__device__ __forceinline__ f4_t mfma(const u4_t a, const u4_t b, const f4_t c) {
  if constexpr (BF16OP)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
}

// Round an fp32 value to 16 bits and back.
template <bool BF16OP> __device__ __forceinline__ uint32_t to_op_bits(float v) {
  if constexpr (BF16OP) return __builtin_bit_cast(uint16_t, (__bf16)v);
  else return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <bool BF16OP> __device__ __forceinline__ float op_bits_to_float(uint32_t h) {
  if constexpr (BF16OP) return __builtin_bit_cast(float, h << 16);
  else return half_bits_to_float(h);
}

// Global-memory pointers: loads through them are global_load (vmcnt only), never flat.
#define QLIN_GLOBAL __attribute__((address_space(1)))
template <typename T> using gptr = T QLIN_GLOBAL*;

// Zero-filled device memory that masked-off lanes load from, so that every path through the
// tile loader issues the same loads (the compiler's wait counting stays exact across tiles).
// 1 KiB: every per-step offset of a tile's loads (at most 8 steps of 64 bytes plus a lane's
// 48) stays inside it.
static __device__ __attribute__((aligned(64))) uint32_t g_zero16[256];

// Pick one of two pointers without indexing the kernel-argument struct by a per-lane value
// (that would turn into a vector load of the pointer and a full memory wait).
template <typename P>
__device__ __forceinline__ gptr<P> pick(P* a, P* b, int second) {
  const uintptr_t ua = reinterpret_cast<uintptr_t>(a), ub = reinterpret_cast<uintptr_t>(b);
  return reinterpret_cast<gptr<P>>(ua + (uintptr_t)second * (ub - ua));
}

__device__ __forceinline__ void store_out(void* y, int dtype, long idx, float v) {
  if (dtype == 0) reinterpret_cast<float*>(y)[idx] = v;
  else if (dtype == 1) reinterpret_cast<_Float16*>(y)[idx] = (_Float16)v;
  else reinterpret_cast<__bf16*>(y)[idx] = (__bf16)v;
}


// Group sums of operands reach 64 * 2^15; they enter the bias MFMA scaled by 2^-kGsumShift.
constexpr int kGsumShift = 7;
// 8-element pieces one thread stages (a chunk holds at most kThreads * kPieceMax pieces).
constexpr int kPieceMax = 12;
// Padding of a staged operand row in LDS (elements), against bank conflicts between rows.
constexpr int kRowPad = 8;
// LDS header: LN sums S1, S2 of up to 32 rows, one scale exponent per operand row, and the
// maximum |value| of each source row (34 at most) during staging.
constexpr int kStatFloats = 64;
constexpr int kExpInts = 128;
constexpr int kRowMax = 64;
constexpr int kHeaderBytes = (kStatFloats + kExpInts + kRowMax) * 4;
// Largest dynamic LDS a launch may ask for (gfx950 has 160 KiB per CU).
constexpr int kLdsMax = 160 * 1024;

__host__ __device__ constexpr int op_pitch(int kc) { return kc + kRowPad; }
// Bytes of the region holding the staged operand rows, their group sums and the per-group
// LN partial sums of the (at most 32) activation rows.
__host__ __device__ constexpr long staging_bytes(int rows, int kc) {
  return (long)rows * op_pitch(kc) * 2 + (long)rows * (kc / 64) * 4 + 32L * (kc / 64) * 2 * 4;
}
// Bytes of the region holding the double-buffered per-wave partial tiles.
__host__ __device__ constexpr long merge_bytes(int mt) { return 2L * kWaves * mt * 256 * 4; }

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global memory, which
// makes every wave wait for its in-flight weight prefetch at each tile; nothing in this
// kernel communicates through global memory, so the LDS fence is all that is needed.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Output slot of thread tid for a tile: outputs 0..63 go to wave (tile mod 8), so the
// epilogue work rotates over the waves instead of always landing on wave 0.
__device__ __forceinline__ int out_slot(int tid, int tile) {
  return (tid + kThreads - 64 * (tile % kWaves)) % kThreads;
}

// Wave-wide fixed-order reductions (xor butterfly over all 64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Unpack a 16-byte piece of 8 16-bit elements.
__device__ __forceinline__ void unpack8(const u4_t raw, int dtype, float v[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = elem_to_float((raw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu, dtype);
}

template <int BITS, bool BF16OP, int MT>
struct Fused {
  static constexpr int NM = Fmt<BITS>::kMfma;
  static constexpr int NG = Fmt<BITS>::kGroups > 0 ? Fmt<BITS>::kGroups : 1;
  static constexpr bool QUANT = BITS != 16;
  static constexpr int STEPK = Fmt<BITS>::kStepK;
  static constexpr int MAXS = max_steps_for(NM, MT);

  u4_t afrag[MAXS][NM][MT];   // operand fragments of this wave's K slice
  u4_t gfrag[MT];             // quantized: group sums of this wave's slice as an A operand
  float unscale[MT][4];       // 2^-e of C rows 4c+v

  // ---- staging: source rows -> operand rows in LDS ----------------------------------
  // Source row rho: rho < T is x row rho; with LN, rho == T is gamma and T + 1 is beta.
  // Operand rows: terms*t + term for activation row t, then gamma (terms*T), beta (+1).
  // All threads share the (row, 8-element piece) pairs of the chunk: thread tid takes pieces
  // tid, tid + kThreads, ...; the 8 pieces of a 64-wide group sit in 8 consecutive lanes.
  // Pass 1 loads every piece, takes the row maxima (LDS atomicMax on the bit pattern of a
  // non-negative float: order-independent) and the per-group shifted LN sums; pass 2
  // converts with the row's power-of-two scale and writes the operand rows and group sums.
  __device__ __forceinline__ static void stage(const LinParams& p, float* stat, int* ex, unsigned* rowmax, float* spart,
                                               uint16_t* op, float* gsum, int kc0, int kc, bool stats, int tid) {
    constexpr int NT = BF16OP ? 3 : 2;          // terms the operand type can need
    const int T = p.T, terms = p.terms;
    const int srows = T + (p.ln ? 2 : 0);
    const int ppr = kc / 8;                     // pieces per row (a multiple of 8)
    const int total = srows * ppr;
    const int pitch = op_pitch(kc);
    const int gpr = kc / 64;
    const uint16_t* x16 = reinterpret_cast<const uint16_t*>(p.x);
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(p.gamma);
    const uint16_t* b16 = reinterpret_cast<const uint16_t*>(p.beta);
    u4_t raw[kPieceMax], graw[kPieceMax];
#pragma unroll
    for (int u = 0; u < kPieceMax; ++u) {
      const int idx = tid + kThreads * u;
      if (idx < total) {
        const int row = idx / ppr, pc = idx - (idx / ppr) * ppr;
        const bool act = row < T;
        const gptr<const uint16_t> src = pick(act ? x16 : g16, b16, (!act && row != T) ? 1 : 0) +
                                         (act ? (long)row * p.K : 0) + kc0 + 8 * pc;
        raw[u] = *reinterpret_cast<gptr<const u4_t>>(src);
        if (act && p.ln) graw[u] = *reinterpret_cast<gptr<const u4_t>>(pick(g16, g16, 0) + kc0 + 8 * pc);
      }
    }
    // pass 1
#pragma unroll
    for (int u = 0; u < kPieceMax; ++u) {
      const int idx = tid + kThreads * u;
      if (kThreads * u < total) {                      // uniform: some lane of the block is live
        const bool live = idx < total;
        const int row = live ? idx / ppr : 0, pc = idx - row * ppr;
        const bool mulg = row < T && p.ln;
        const float x0 = mulg ? elem_to_float(x16[(long)row * p.K], p.x_dtype) : 0.0f;
        float a[8], g[8];
        unpack8(raw[u], p.x_dtype, a);
        unpack8(graw[u], p.x_dtype, g);
        float amax = 0.0f, s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float d = a[jj] - x0;
          amax = fmaxf(amax, fabsf(mulg ? d * g[jj] : a[jj]));
          s1 += d;
          s2 += d * d;
        }
        if (live) atomicMax(rowmax + row, __builtin_bit_cast(unsigned, amax));
        if (p.ln && stats) {
          s1 += __shfl_xor(s1, 1); s1 += __shfl_xor(s1, 2); s1 += __shfl_xor(s1, 4);
          s2 += __shfl_xor(s2, 1); s2 += __shfl_xor(s2, 2); s2 += __shfl_xor(s2, 4);
          if (live && mulg && (pc & 7) == 0) { spart[(row * gpr + pc / 8) * 2] = s1; spart[(row * gpr + pc / 8) * 2 + 1] = s2; }
        }
      }
    }
    lds_barrier();
    // pass 2
#pragma unroll
    for (int u = 0; u < kPieceMax; ++u) {
      const int idx = tid + kThreads * u;
      if (kThreads * u < total) {
        const bool live = idx < total;
        const int row = live ? idx / ppr : 0, pc = idx - row * ppr;
        const bool act = row < T;
        const bool mulg = act && p.ln;
        const float x0 = mulg ? elem_to_float(x16[(long)row * p.K], p.x_dtype) : 0.0f;
        const float amax = __builtin_bit_cast(float, rowmax[row]);
        const bool need = act ? p.scale_act : p.scale_gb;
        int e = 0;
        if (need && amax > 0.0f && amax < __builtin_inff()) {
          e = 14 - ilogbf(amax);
          e = e > 126 ? 126 : (e < -126 ? -126 : e);
        }
        const float scl = ldexpf(1.0f, e);
        const int r0 = act ? terms * row : terms * T + (row - T);
        const int nterm = act ? terms : 1;
        if (live && pc == 0)
          for (int term = 0; term < nterm; ++term) ex[r0 + term] = e;
        float a[8], g[8];
        unpack8(raw[u], p.x_dtype, a);
        unpack8(graw[u], p.x_dtype, g);
        uint32_t el[NT][8];
        float ts[NT];
#pragma unroll
        for (int term = 0; term < NT; ++term) ts[term] = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int kj = slot_k<BITS>(jj);
          const float v = mulg ? (a[kj] - x0) * g[kj] : a[kj];
          const float sv = v * scl;
          if constexpr (BF16OP) {
            const uint32_t hi = to_op_bits<true>(sv);
            const float r1 = sv - op_bits_to_float<true>(hi);
            const uint32_t mid = to_op_bits<true>(r1);
            const uint32_t lo = to_op_bits<true>(r1 - op_bits_to_float<true>(mid));
            el[0][jj] = hi; el[1][jj] = mid; el[2][jj] = lo;
          } else {
            const uint32_t hi = to_op_bits<false>(sv);
            el[0][jj] = hi;
            el[1][jj] = to_op_bits<false>(sv - op_bits_to_float<false>(hi));
          }
#pragma unroll
          for (int term = 0; term < NT; ++term) ts[term] += op_bits_to_float<BF16OP>(el[term][jj]);
        }
#pragma unroll
        for (int term = 0; term < NT; ++term) {
          if (term < nterm && live) {
            u4_t w;
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = el[term][2 * r] | (el[term][2 * r + 1] << 16);
            *reinterpret_cast<u4_t*>(op + (long)(r0 + term) * pitch + 8 * pc) = w;
          }
        }
        if constexpr (QUANT) {
#pragma unroll
          for (int term = 0; term < NT; ++term) {
            float t = ts[term];
            t += __shfl_xor(t, 1);
            t += __shfl_xor(t, 2);
            t += __shfl_xor(t, 4);
            if (term < nterm && live && (pc & 7) == 0) gsum[(r0 + term) * gpr + pc / 8] = t;
          }
        }
      }
    }
    // LayerNorm sums of each activation row, in group order
    if (p.ln && stats && tid < T) {
      float s1 = 0.0f, s2 = 0.0f;
      for (int g = 0; g < gpr; ++g) { s1 += spart[(tid * gpr + g) * 2]; s2 += spart[(tid * gpr + g) * 2 + 1]; }
      stat[2 * tid] += s1;
      stat[2 * tid + 1] += s2;
    }
  }

  // ---- per-wave fragment load from the staged rows ----------------------------------
  __device__ __forceinline__ void load_frags(const LinParams& p, const int* ex, const uint16_t* op, const float* gsum,
                                             int kc0, int kc, int cs0, int s_lo, int nsw, int c, int li) {
    const int R = p.rows, pitch = op_pitch(kc), gpr = kc / 64;
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
#pragma unroll
      for (int q = 0; q < NM; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = 16 * mt + li;
          const int kk = (s_lo + s) * STEPK + frag_base<BITS>(q, c) - kc0;
          u4_t a = (u4_t){0u, 0u, 0u, 0u};
          if (s < nsw && r < R && kk < kc) a = *reinterpret_cast<const u4_t*>(op + (long)r * pitch + kk);
          afrag[s][q][mt] = a;
        }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * mt + 4 * c + v;
        unscale[mt][v] = r < R ? ldexpf(1.0f, -ex[r]) : 1.0f;
      }
      if constexpr (QUANT) {
        const int r = 16 * mt + li;
        uint32_t el[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gi = 8 * (c & 1) + j;
          const int gl = (s_lo - cs0) * NG + gi;
          float v = 0.0f;
          if (r < R && gi < nsw * NG && gl < gpr) v = gsum[r * gpr + gl] * (1.0f / (float)(1 << kGsumShift));
          const uint32_t hi = to_op_bits<false>(v);
          const uint32_t lo = to_op_bits<false>(v - op_bits_to_float<false>(hi));
          el[j] = (c >> 1) ? lo : hi;
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) gfrag[mt][w] = el[2 * w] | (el[2 * w + 1] << 16);
      }
    }
  }

  // Lane (c, li) of a tile: weight row (projection, n) it streams.
  __device__ __forceinline__ static void tile_row(const LinParams& p, int tile, int li, int& proj, int& n) {
    if (p.gateup) { proj = li >> 3; n = tile * 8 + (li & 7); }
    else { proj = 0; n = tile * 16 + li; }
  }

  // Registers a tile's loads land in.  Loaded values are not combined here: consuming one
  // would make the compiler wait for every load issued before it, the prefetch included.
  struct TileRegs {
    u4_t dw[MAXS];          // 16 code bytes per step
    uint32_t sc[MAXS];      // fp16 scale bits of the step's groups, packed (group g in bits 16g)
    uint32_t bi[MAXS];      // fp16 bias bits, packed the same way
  };

  // Epilogue inputs of the output this thread finishes, out_slot(tid, tile) = (t, col):
  // residual[t, n] and constant[n] of a linear tile (zeros when absent or out of range).
  struct EpiRegs {
    uint16_t res, add;
  };
  __device__ __forceinline__ static void load_epi(const LinParams& p, int tile, EpiRegs& e) {
    const gptr<const uint16_t> z16 = pick(reinterpret_cast<const uint16_t*>(g_zero16),
                                          reinterpret_cast<const uint16_t*>(g_zero16), 0);
    const int q = out_slot(threadIdx.x, tile);
    const int t = q >> 4, on = tile * 16 + (q & 15);
    const bool mine = !p.gateup && tile < p.ntiles && t < p.T && on < p.N;
    const gptr<const uint16_t> rp = pick(reinterpret_cast<const uint16_t*>(p.res), reinterpret_cast<const uint16_t*>(p.res), 0);
    const gptr<const uint16_t> ap = pick(reinterpret_cast<const uint16_t*>(p.add), reinterpret_cast<const uint16_t*>(p.add), 0);
    e.res = *((mine && p.res) ? rp + (long)t * p.N + on : z16);
    e.add = *((mine && p.add) ? ap + on : z16);
  }

  // Issue the loads of a tile's codes, scales and biases for steps [s_lo, s_lo + nsw).
  // One base address per lane and tile, then immediate offsets per step.  A lane with no
  // row (n >= N, or a tile past the last) streams from the zero buffer instead, so every
  // tile issues the same loads; steps >= nsw (uniform) are skipped.  Rows must consist of
  // whole 64-byte steps (4-bit K = 64 mod 128 goes through the chunked variant).
  template <bool CHECKED = false>
  __device__ __forceinline__ static void load_tile(const LinParams& p, int tile, int s_lo, int nsw, int c, int li,
                                                   TileRegs& r) {
    int proj, n;
    tile_row(p, tile, li, proj, n);
    const bool valid = tile < p.ntiles && n < p.N;
    const long row_bytes = (long)p.K * BITS / 8;
    const int G = p.K / 64;
    const gptr<const char> zero = pick(reinterpret_cast<const char*>(g_zero16), reinterpret_cast<const char*>(g_zero16), 0);
    const gptr<const char> wb = pick(reinterpret_cast<const char*>(p.w[0]), reinterpret_cast<const char*>(p.w[1]), proj);
    __builtin_amdgcn_sched_barrier(0);
    const gptr<const char> cb = valid ? wb + (long)n * row_bytes + (long)s_lo * 64 + 16 * c : zero + 16 * c;
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      // steps >= nsw (uniform) read the zero buffer: no branch, so the whole batch issues
      // back to back and the wait counts stay exact
      const gptr<const char> a = s < nsw ? cb + s * 64 : zero + 16 * c;
      if constexpr (CHECKED) {   // a row may end half-way through its last step
        const bool in = (long)(s_lo + s) * 64 + 16 * c < row_bytes;
        r.dw[s] = *reinterpret_cast<gptr<const u4_t>>(in ? a : zero + 16 * c);
      } else {
        r.dw[s] = *reinterpret_cast<gptr<const u4_t>>(a);
      }
    }
    if constexpr (QUANT) {
      // A step's scales (biases) are NG consecutive fp16 values: 4-bit steps load them as one
      // aligned dword (K is a multiple of 128 here, so n*G + 2*s is even), 8-bit as a ushort.
      // They stay packed until compute_tile; splitting them here would make the compiler wait.
      const gptr<const uint16_t> zh = pick(reinterpret_cast<const uint16_t*>(g_zero16),
                                           reinterpret_cast<const uint16_t*>(g_zero16), 0);
      const long go = (long)n * G + (long)s_lo * NG;
      const gptr<const uint16_t> sbase = valid ? pick(p.sc[0], p.sc[1], proj) + go : zh;
      const gptr<const uint16_t> bbase = valid ? pick(p.bi[0], p.bi[1], proj) + go : zh;
#pragma unroll
      for (int s = 0; s < MAXS; ++s) {
        const bool live = s < nsw;
        if constexpr (CHECKED) {
          // rows may end half-way through a step: fetch each group on its own
          uint32_t sv = 0u, bv = 0u;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const bool in = live && (s_lo + s) * NG + g < G;
            sv |= (uint32_t)*(in ? sbase + s * NG + g : zh) << (16 * g);
            bv |= (uint32_t)*(in ? bbase + s * NG + g : zh) << (16 * g);
          }
          r.sc[s] = sv;
          r.bi[s] = bv;
        } else if constexpr (NG == 2) {
          r.sc[s] = *reinterpret_cast<gptr<const uint32_t>>(live ? sbase + 2 * s : zh);
          r.bi[s] = *reinterpret_cast<gptr<const uint32_t>>(live ? bbase + 2 * s : zh);
        } else {
          r.sc[s] = *(live ? sbase + s : zh);
          r.bi[s] = *(live ? bbase + s : zh);
        }
      }
    }
    // keep the batch together: nothing from the surrounding compute moves in between
    __builtin_amdgcn_sched_barrier(0);
  }

  // Stream one tile's loaded codes through the fragments into acc.
  __device__ __forceinline__ void compute_tile(int nsw, int c, const TileRegs& r, f4_t acc[MT]) {
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      if (s < nsw) {
        u4_t d = r.dw[s];
        if constexpr (BITS == 4) {
          const auto r01 = __builtin_amdgcn_permlane32_swap(d[0], d[1], false, false);
          const auto r23 = __builtin_amdgcn_permlane32_swap(d[2], d[3], false, false);
          d[0] = r01[0]; d[1] = r01[1]; d[2] = r23[0]; d[3] = r23[1];
        }
        if constexpr (QUANT) {
          // every group's partial first (independent accumulators), then the scale FMAs
          f4_t cg[NG][MT];
#pragma unroll
          for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) cg[g][mt] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int qq = 0; qq < NM / NG; ++qq)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              const int q = g * (NM / NG) + qq;
              const u4_t b = convert_codes<BITS>(d, q);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) cg[g][mt] = mfma<BF16OP>(afrag[s][q][mt], b, cg[g][mt]);
            }
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const float sf = half_bits_to_float((r.sc[s] >> (16 * g)) & 0xFFFFu);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[mt][v] = fmaf(sf, cg[g][mt][v], acc[mt][v]);
          }
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma<BF16OP>(afrag[s][0][mt], d, acc[mt]);
        }
      } else {
        // unused step: still read its (zero) registers, so that no path leaves a load unread
        // (the compiler would drain every outstanding load, the prefetch too, before reusing them)
        asm volatile("" ::"v"(r.dw[s]), "v"(r.sc[s]), "v"(r.bi[s]));
      }
    }
    if constexpr (QUANT) {
      // sum_g b[n, g] * (sum of group g's operands): one MFMA per row tile
      // slot j of lane group c is the bias of this wave's group 8*(c&1) + j
      uint32_t el[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // groups past this wave's slice get 0 (their loads were skipped)
        const uint32_t lo = (j < MAXS * NG && j < nsw * NG) ? (r.bi[j / NG] >> (16 * (j % NG))) & 0xFFFFu : 0u;
        const uint32_t hi = (8 + j < MAXS * NG && 8 + j < nsw * NG)
                                ? (r.bi[(8 + j) / NG] >> (16 * ((8 + j) % NG))) & 0xFFFFu : 0u;
        el[j] = (c & 1) ? hi : lo;
      }
      u4_t bfr;
#pragma unroll
      for (int w = 0; w < 4; ++w) bfr[w] = el[2 * w] | (el[2 * w + 1] << 16);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f4_t cb = mfma<false>(gfrag[mt], bfr, (f4_t){0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mt][v] = fmaf(cb[v], (float)(1 << kGsumShift), acc[mt][v]);
      }
    }
  }
};

// Sum over the workgroup's waves of C row r, column col, from the LDS partials.
template <int MT>
__device__ __forceinline__ float merged(const float* red, int buf, int r, int col) {
  const int lane = 16 * ((r & 15) >> 2) + col;
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[((buf * kWaves + w) * MT + (r >> 4)) * 256 + lane * 4 + (r & 3)];
  return s;
}

// Output value before the epilogue: no LN, the sum of the row's terms; with LN the fold
// rstd * (P - m G) + B, m = S1 / K and var = S2 / K - m^2 (biased, clamped at 0).
template <int MT>
__device__ __forceinline__ float folded(const LinParams& p, const float* red, const float* stat, int buf, int t, int col) {
  const int terms = p.terms;
  float P = 0.0f;
  for (int term = 0; term < terms; ++term) P += merged<MT>(red, buf, terms * t + term, col);
  if (!p.ln) return P;
  const float Gw = merged<MT>(red, buf, terms * p.T, col);
  const float Bw = merged<MT>(red, buf, terms * p.T + 1, col);
  const float m = stat[2 * t] / (float)p.K;
  const float var = fmaxf(stat[2 * t + 1] / (float)p.K - m * m, 0.0f);
  const float rstd = 1.0f / sqrtf(var + p.eps);
  return rstd * (P - m * Gw) + Bw;
}

// Epilogue and store of one tile ([p1] `_linear_kernel`: GELU, then residual, then constant).
// Thread tid finishes output slot out_slot(tid, tile).
template <int MT>
__device__ __forceinline__ void finalize(const LinParams& p, const float* red, const float* stat, int buf, int tile, int tid,
                                         uint32_t res_bits, uint32_t add_bits) {
  tid = out_slot(tid, tile);
  if (!p.gateup) {
    if (tid < p.T * 16) {
      const int t = tid >> 4, col = tid & 15, n = tile * 16 + col;
      if (n < p.N) {
        float v = folded<MT>(p, red, stat, buf, t, col);
        if (p.act == 1) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
        if (p.res) v += elem_to_float(res_bits, p.x_dtype);
        if (p.add) v += elem_to_float(add_bits, p.x_dtype);
        store_out(p.y, p.y_dtype, (long)t * p.N + n, v);
      }
    }
  } else {
    if (tid < p.T * 8) {
      const int t = tid >> 3, j = tid & 7, n = tile * 8 + j;
      if (n < p.N) {
        const float g = folded<MT>(p, red, stat, buf, t, j);
        const float u = folded<MT>(p, red, stat, buf, t, j + 8);
        store_out(p.y, p.y_dtype, (long)t * p.N + n, g / (1.0f + expf(-g)) * u);
      }
    }
  }
}

template <int BITS, bool BF16OP, int MT, bool CHUNKED>
__global__ __launch_bounds__(kThreads) void fused_kernel(const LinParams p) {
  using S = Fused<BITS, BF16OP, MT>;
  constexpr int STEPK = S::STEPK;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  float* stat = reinterpret_cast<float*>(lds_raw);
  int* ex = reinterpret_cast<int*>(lds_raw + kStatFloats * 4);
  unsigned* rowmax = reinterpret_cast<unsigned*>(lds_raw + (kStatFloats + kExpInts) * 4);
  unsigned char* region = lds_raw + kHeaderBytes;
  float* red = reinterpret_cast<float*>(region);

  const int tid = threadIdx.x, lane = tid & 63, c = lane >> 4, li = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  auto slice = [&](int ch, int& cs0, int& s_lo, int& nsw) {
    cs0 = ch * p.chunk_steps;
    const int sc = min(p.chunk_steps, p.steps - cs0);
    s_lo = cs0 + (wv * sc) / kWaves;
    nsw = cs0 + ((wv + 1) * sc) / kWaves - s_lo;
  };
  // Stage chunk ch into LDS and load this wave's fragments from it.
  S st;
  auto prepare = [&](int ch, bool stats, int& cs0, int& s_lo, int& nsw) {
    slice(ch, cs0, s_lo, nsw);
    const int kc0 = cs0 * STEPK;
    const int kc = min(p.chunk_steps * STEPK, p.K - kc0);
    uint16_t* op = reinterpret_cast<uint16_t*>(region);
    float* gsum = reinterpret_cast<float*>(region + (long)p.rows * op_pitch(kc) * 2);
    float* spart = gsum + (long)p.rows * (kc / 64);
    if (tid < kRowMax) rowmax[tid] = 0u;
    lds_barrier();
    S::stage(p, stat, ex, rowmax, spart, op, gsum, kc0, kc, stats, tid);
    lds_barrier();
    st.load_frags(p, ex, op, gsum, kc0, kc, cs0, s_lo, nsw, c, li);
    lds_barrier();
  };
  // Merge the waves' partials of a tile in LDS (double-buffered by tile parity), finish it.
  auto merge_finish = [&](const f4_t acc[MT], int tile, int buf, const typename S::EpiRegs& e) {
    float* rb = red + (buf * kWaves + wv) * MT * 256;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f4_t v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = acc[mt][j] * st.unscale[mt][j];
      *reinterpret_cast<f4_t*>(rb + mt * 256 + lane * 4) = v;
    }
    // Every lane reads its residual and constant here, used or not: a loaded register left
    // unread on some path makes the compiler drain all loads (the prefetch too) before the
    // register is reused.
    const uint32_t res_bits = e.res, add_bits = e.add;
    asm volatile("" ::"v"(res_bits), "v"(add_bits));
    lds_barrier();
    finalize<MT>(p, red, stat, buf, tile, tid, res_bits, add_bits);
  };

  if (tid < kStatFloats) stat[tid] = 0.0f;
  lds_barrier();

  int cs0, s_lo, nsw;
  if constexpr (!CHUNKED) {
    // All of K fits: build the fragments once, then stream tiles with the next tile's loads
    // always in flight.  Two register sets alternate (no copy at the end of an iteration,
    // which would make the compiler wait for the prefetch).
    slice(0, cs0, s_lo, nsw);
    typename S::TileRegs ra, rb;
    int tile = blockIdx.x;
    S::load_tile(p, tile, s_lo, nsw, c, li, ra);   // the weight stream starts before staging
    prepare(0, true, cs0, s_lo, nsw);
    int buf = 0;
    for (;;) {
      // epilogue inputs are loaded and used within one half: a load still in flight across
      // the loop edge would make the compiler drain the prefetch at the top of the loop
      typename S::EpiRegs e;
      S::load_epi(p, tile, e);
      const int t1 = tile + gridDim.x;
      S::load_tile(p, t1, s_lo, nsw, c, li, rb);   // past the last tile this loads zeros
      {
        f4_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
        st.compute_tile(nsw, c, ra, acc);
        merge_finish(acc, tile, buf, e);
      }
      tile = t1;
      buf ^= 1;
      if (tile >= p.ntiles) break;
      S::load_epi(p, tile, e);
      const int t2 = tile + gridDim.x;
      S::load_tile(p, t2, s_lo, nsw, c, li, ra);
      {
        f4_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
        st.compute_tile(nsw, c, rb, acc);
        merge_finish(acc, tile, buf, e);
      }
      tile = t2;
      buf ^= 1;
      if (tile >= p.ntiles) break;
    }
  } else {
    // Long K: rebuild the fragments per chunk.  acc stays in the current chunk's scaled
    // units; switching chunks multiplies by a ratio of powers of two (exact).
    const int nchunks = (p.steps + p.chunk_steps - 1) / p.chunk_steps;
    bool first = true;
    int buf = 0;
    for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x, buf ^= 1) {
      f4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
      typename S::TileRegs r;
      for (int ch = 0; ch < nchunks; ++ch) {
        float prev[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) prev[mt][j] = st.unscale[mt][j];
        if (!first || ch > 0) lds_barrier();   // earlier readers of the LDS region are done
        prepare(ch, first, cs0, s_lo, nsw);
        S::template load_tile<true>(p, tile, s_lo, nsw, c, li, r);
        if (ch > 0) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mt][j] *= prev[mt][j] / st.unscale[mt][j];
        }
        st.compute_tile(nsw, c, r, acc);
      }
      first = false;
      typename S::EpiRegs e;
      S::load_epi(p, tile, e);
      merge_finish(acc, tile, buf, e);
    }
  }
}

// Dynamic LDS a launch needs: header + max(staging, merge).
__host__ __device__ constexpr long lds_bytes_for(int rows, int kc, int mt) {
  return kHeaderBytes + (staging_bytes(rows, kc) > merge_bytes(mt) ? staging_bytes(rows, kc) : merge_bytes(mt));
}

template <int BITS, bool BF16OP, int MT, bool CHUNKED>
hipError_t launch_variant(const LinParams& p, int grid, size_t lds, hipStream_t s) {
  // Above 64 KiB of dynamic LDS the kernel must opt in once (a host-side attribute).
  static bool opted_in = false;
  if (!opted_in) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_kernel<BITS, BF16OP, MT, CHUNKED>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e != hipSuccess) return e;
    opted_in = true;
  }
  hipLaunchKernelGGL((fused_kernel<BITS, BF16OP, MT, CHUNKED>), dim3(grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

template <int BITS, bool BF16OP, int MT>
hipError_t launch_one(const LinParams& p, int grid, size_t lds, hipStream_t s) {
  // The streaming variant needs all of K staged at once and rows of whole 64-byte steps.
  const bool whole_steps = ((long)p.K * BITS / 8) % 64 == 0;
  return (p.chunk_steps >= p.steps && whole_steps) ? launch_variant<BITS, BF16OP, MT, false>(p, grid, lds, s)
                                                   : launch_variant<BITS, BF16OP, MT, true>(p, grid, lds, s);
}

}  // namespace qlin
