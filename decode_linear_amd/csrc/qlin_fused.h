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
__device__ __forceinline__ uint32_t nib_lo_to_h2(uint32_t d) {
  const uint32_t h = (d & 0x000F000Fu) | 0x64006400u;
  const h2_t v = __builtin_bit_cast(h2_t, h) - (h2_t){(_Float16)1024.0f, (_Float16)1024.0f};
  return __builtin_bit_cast(uint32_t, v);
}
// Nibbles 1 and 5 (bits 4-7 and 20-23): 1024 + 16 n, scaled back exactly: (1024+16n)/16 - 64.
__device__ __forceinline__ uint32_t nib_hi_to_h2(uint32_t d) {
  const uint32_t h = (d & 0x00F000F0u) | 0x64006400u;
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

__device__ __forceinline__ void store_out(void* y, int dtype, long idx, float v) {
  if (dtype == 0) reinterpret_cast<float*>(y)[idx] = v;
  else if (dtype == 1) reinterpret_cast<_Float16*>(y)[idx] = (_Float16)v;
  else reinterpret_cast<__bf16*>(y)[idx] = (__bf16)v;
}


// Group sums of operands reach 64 * 2^15; they enter the bias MFMA scaled by 2^-kGsumShift.
constexpr int kGsumShift = 7;
// 8-element pieces of one staged row per lane (so a chunk spans at most 8*64*8 = 4096 k).
constexpr int kPieceMax = 8;
// Padding of a staged operand row in LDS (elements), against bank conflicts between rows.
constexpr int kRowPad = 8;
// LDS header: LN sums S1, S2 of up to 32 rows, then one scale exponent per operand row.
constexpr int kStatFloats = 64;
constexpr int kExpInts = 128;
constexpr int kHeaderBytes = (kStatFloats + kExpInts) * 4;
// Largest dynamic LDS a launch may ask for (gfx950 has 160 KiB per CU).
constexpr int kLdsMax = 160 * 1024;

__host__ __device__ constexpr int op_pitch(int kc) { return kc + kRowPad; }
// Bytes of the region holding the staged operand rows and their group sums.
__host__ __device__ constexpr long staging_bytes(int rows, int kc) {
  return (long)rows * op_pitch(kc) * 2 + (long)rows * (kc / 64) * 4;
}
// Bytes of the region holding the double-buffered per-wave partial tiles.
__host__ __device__ constexpr long merge_bytes(int mt) { return 2L * kWaves * mt * 256 * 4; }

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
  // Round r: wave w stages source row 8r + w; lane l holds pieces l, l + 64, ... (8 k each).
  __device__ __forceinline__ static void stage(const LinParams& p, float* stat, int* ex, uint16_t* op, float* gsum,
                                               int kc0, int kc, bool stats, int wv, int lane) {
    constexpr int NT = BF16OP ? 3 : 2;          // terms the operand type can need
    const int T = p.T, terms = p.terms;
    const int srows = T + (p.ln ? 2 : 0);
    const int ppr = kc / 8;                     // pieces per row (a multiple of 8)
    const int pitch = op_pitch(kc);
    const int gpr = kc / 64;
    for (int rho = wv; rho < srows; rho += kWaves) {
      const bool act = rho < T;
      const bool mulg = act && p.ln;
      const uint16_t* src = reinterpret_cast<const uint16_t*>(act ? p.x : (rho == T ? p.gamma : p.beta)) +
                            (act ? (long)rho * p.K : 0) + kc0;
      const uint16_t* gam = reinterpret_cast<const uint16_t*>(p.gamma) + kc0;
      u4_t raw[kPieceMax], graw[kPieceMax];
#pragma unroll
      for (int u = 0; u < kPieceMax; ++u) {
        const int pc = lane + 64 * u;
        raw[u] = (u4_t){0u, 0u, 0u, 0u};
        graw[u] = (u4_t){0u, 0u, 0u, 0u};
        if (pc < ppr) {
          raw[u] = *reinterpret_cast<const u4_t*>(src + 8 * pc);
          if (mulg) graw[u] = *reinterpret_cast<const u4_t*>(gam + 8 * pc);
        }
      }
      const float x0 = mulg ? elem_to_float(reinterpret_cast<const uint16_t*>(p.x)[(long)rho * p.K], p.x_dtype) : 0.0f;
      // The passes below walk the pieces one per iteration (not unrolled, to bound register
      // use) and rotate the arrays by one slot each time; after kPieceMax steps they are back.
      auto rotate = [&]() {
        const u4_t r0 = raw[0], g0 = graw[0];
#pragma unroll
        for (int i = 0; i + 1 < kPieceMax; ++i) { raw[i] = raw[i + 1]; graw[i] = graw[i + 1]; }
        raw[kPieceMax - 1] = r0;
        graw[kPieceMax - 1] = g0;
      };
      // pass 1: row max (for the scale) and the shifted LayerNorm sums
      float amax = 0.0f, s1 = 0.0f, s2 = 0.0f;
#pragma unroll 1
      for (int u = 0; u < kPieceMax; ++u) {
        if (lane + 64 * u < ppr) {
          float a[8], g[8];
          unpack8(raw[0], p.x_dtype, a);
          unpack8(graw[0], p.x_dtype, g);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float d = a[jj] - x0;
            const float v = mulg ? d * g[jj] : a[jj];
            amax = fmaxf(amax, fabsf(v));
            if (mulg) { s1 += d; s2 += d * d; }
          }
        }
        rotate();
      }
      amax = wave_max(amax);
      if (mulg && stats) {
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        if (lane == 0) { stat[2 * rho] += s1; stat[2 * rho + 1] += s2; }
      }
      const bool need = act ? p.scale_act : p.scale_gb;
      int e = 0;
      if (need && amax > 0.0f && amax < __builtin_inff()) {
        e = 14 - ilogbf(amax);
        e = e > 126 ? 126 : (e < -126 ? -126 : e);
      }
      const float scl = ldexpf(1.0f, e);
      const int r0 = act ? terms * rho : terms * T + (rho - T);
      const int nterm = act ? terms : 1;
      if (lane == 0)
        for (int term = 0; term < nterm; ++term) ex[r0 + term] = e;
      // pass 2: operand terms in MFMA slot order, and their per-group sums
#pragma unroll 1
      for (int u = 0; u < kPieceMax; ++u) {
        const int pc = lane + 64 * u;
        const bool live = pc < ppr;
        float a[8], g[8];
        unpack8(raw[0], p.x_dtype, a);
        unpack8(graw[0], p.x_dtype, g);
        rotate();
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
          // the 8 pieces of a group sit in 8 consecutive lanes
#pragma unroll
          for (int term = 0; term < NT; ++term) {
            float t = ts[term];
            t += __shfl_xor(t, 1);
            t += __shfl_xor(t, 2);
            t += __shfl_xor(t, 4);
            if (term < nterm && live && (lane & 7) == 0) gsum[(r0 + term) * gpr + pc / 8] = t;
          }
        }
      }
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

  // Issue the loads of a tile's codes, scales and biases for steps [s_lo, s_lo + nsw).
  __device__ __forceinline__ static void load_tile(const LinParams& p, int tile, int s_lo, int nsw, int c, int li,
                                                   u4_t dw[MAXS], uint32_t sb[MAXS], u4_t& bfr) {
    int proj, n;
    tile_row(p, tile, li, proj, n);
    const bool valid = n < p.N;
    const long row_bytes = (long)p.K * BITS / 8;
    const char* wrow = reinterpret_cast<const char*>(p.w[proj]) + (long)n * row_bytes;
    const int G = p.K / 64;
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      dw[s] = (u4_t){0u, 0u, 0u, 0u};
      const long off = (long)(s_lo + s) * 64 + 16 * c;
      if (s < nsw && valid && off < row_bytes) dw[s] = *reinterpret_cast<const u4_t*>(wrow + off);
      if constexpr (QUANT) {
        sb[s] = 0u;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int grp = (s_lo + s) * NG + g;
          if (s < nsw && valid && grp < G) sb[s] |= (uint32_t)p.sc[proj][(long)n * G + grp] << (16 * g);
        }
      }
    }
    if constexpr (QUANT) {
      // B operand of the bias product: slot j of lane group c = bias of group 8*(c&1) + j
      uint32_t el[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gi = 8 * (c & 1) + j;
        const int grp = s_lo * NG + gi;
        el[j] = (valid && gi < nsw * NG && grp < G) ? (uint32_t)p.bi[proj][(long)n * G + grp] : 0u;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) bfr[r] = el[2 * r] | (el[2 * r + 1] << 16);
    }
  }

  // Stream one tile's loaded codes through the fragments into acc.
  __device__ __forceinline__ void compute_tile(int nsw, const u4_t dw[MAXS], const uint32_t sb[MAXS], const u4_t bfr,
                                               f4_t acc[MT]) {
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      if (s < nsw) {
        u4_t d = dw[s];
        if constexpr (BITS == 4) {
          const auto r01 = __builtin_amdgcn_permlane32_swap(d[0], d[1], false, false);
          const auto r23 = __builtin_amdgcn_permlane32_swap(d[2], d[3], false, false);
          d[0] = r01[0]; d[1] = r01[1]; d[2] = r23[0]; d[3] = r23[1];
        }
        if constexpr (QUANT) {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            f4_t cg[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) cg[mt] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int qq = 0; qq < NM / NG; ++qq) {
              const int q = g * (NM / NG) + qq;
              const u4_t b = convert_codes<BITS>(d, q);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) cg[mt] = mfma<BF16OP>(afrag[s][q][mt], b, cg[mt]);
            }
            const float sf = half_bits_to_float((sb[s] >> (16 * g)) & 0xFFFFu);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[mt][v] = fmaf(sf, cg[mt][v], acc[mt][v]);
          }
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma<BF16OP>(afrag[s][0][mt], d, acc[mt]);
        }
      }
    }
    if constexpr (QUANT) {
      // sum_g b[n, g] * (sum of group g's operands): one MFMA per row tile
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
template <int MT>
__device__ __forceinline__ void finalize(const LinParams& p, const float* red, const float* stat, int buf, int tile, int tid) {
  if (!p.gateup) {
    if (tid < p.T * 16) {
      const int t = tid >> 4, col = tid & 15, n = tile * 16 + col;
      if (n < p.N) {
        float v = folded<MT>(p, red, stat, buf, t, col);
        if (p.act == 1) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
        if (p.res) v += elem_to_float(reinterpret_cast<const uint16_t*>(p.res)[(long)t * p.N + n], p.x_dtype);
        if (p.add) v += elem_to_float(reinterpret_cast<const uint16_t*>(p.add)[n], p.x_dtype);
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

template <int BITS, bool BF16OP, int MT>
__global__ __launch_bounds__(kThreads) void fused_kernel(const LinParams p) {
  using S = Fused<BITS, BF16OP, MT>;
  constexpr int MAXS = S::MAXS;
  constexpr int STEPK = S::STEPK;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  float* stat = reinterpret_cast<float*>(lds_raw);
  int* ex = reinterpret_cast<int*>(lds_raw + kStatFloats * 4);
  unsigned char* region = lds_raw + kHeaderBytes;
  float* red = reinterpret_cast<float*>(region);

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, c = lane >> 4, li = lane & 15;
  const int nchunks = (p.steps + p.chunk_steps - 1) / p.chunk_steps;
  const bool single = nchunks == 1;

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
    S::stage(p, stat, ex, op, gsum, kc0, kc, stats, wv, lane);
    __syncthreads();
    st.load_frags(p, ex, op, gsum, kc0, kc, cs0, s_lo, nsw, c, li);
    __syncthreads();
  };

  if (tid < kStatFloats) stat[tid] = 0.0f;
  __syncthreads();

  int cs0, s_lo, nsw;
  slice(0, cs0, s_lo, nsw);
  u4_t cur[MAXS], nxt[MAXS], bfc, bfn;
  uint32_t sbc[MAXS], sbn[MAXS];
  int tile = blockIdx.x;
  if (single) S::load_tile(p, tile, s_lo, nsw, c, li, cur, sbc, bfc);   // the weight stream starts first
  bool first = true;
  int buf = 0;
  for (; tile < p.ntiles; tile += gridDim.x, buf ^= 1) {
    f4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
    // With one chunk the fragments are built once and each tile's loads go out one tile
    // ahead.  Long K rebuilds them per chunk; acc stays in the current chunk's scaled
    // units, and switching chunks multiplies by a ratio of powers of two (exact).
    for (int ch = 0; ch < nchunks; ++ch) {
      if (!single || first) {
        float prev[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) prev[mt][j] = st.unscale[mt][j];
        if (!first) __syncthreads();   // the previous tile's merge has been read
        prepare(ch, first, cs0, s_lo, nsw);
        if (!single) {
          S::load_tile(p, tile, s_lo, nsw, c, li, cur, sbc, bfc);
          if (ch > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[mt][j] *= prev[mt][j] / st.unscale[mt][j];
          }
        }
      }
      if (single) {
        const int next = tile + gridDim.x;
        if (next < p.ntiles) S::load_tile(p, next, s_lo, nsw, c, li, nxt, sbn, bfn);
      }
      st.compute_tile(nsw, cur, sbc, bfc, acc);
    }
    first = false;
    // merge the waves' partials in LDS (double-buffered by tile parity), then finish
    float* rb = red + (buf * kWaves + wv) * MT * 256;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f4_t v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = acc[mt][j] * st.unscale[mt][j];
      *reinterpret_cast<f4_t*>(rb + mt * 256 + lane * 4) = v;
    }
    __syncthreads();
    finalize<MT>(p, red, stat, buf, tile, tid);
    if (single) {
#pragma unroll
      for (int s = 0; s < MAXS; ++s) { cur[s] = nxt[s]; sbc[s] = sbn[s]; }
      bfc = bfn;
    }
  }
}

// Dynamic LDS a launch needs: header + max(staging, merge).
__host__ __device__ constexpr long lds_bytes_for(int rows, int kc, int mt) {
  return kHeaderBytes + (staging_bytes(rows, kc) > merge_bytes(mt) ? staging_bytes(rows, kc) : merge_bytes(mt));
}

template <int BITS, bool BF16OP, int MT>
hipError_t launch_one(const LinParams& p, int grid, size_t lds, hipStream_t s) {
  // Above 64 KiB of dynamic LDS the kernel must opt in once (a host-side attribute).
  static bool opted_in = false;
  if (!opted_in) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_kernel<BITS, BF16OP, MT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e != hipSuccess) return e;
    opted_in = true;
  }
  hipLaunchKernelGGL((fused_kernel<BITS, BF16OP, MT>), dim3(grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace qlin
