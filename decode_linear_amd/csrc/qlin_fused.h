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
//     b, b + grid, ...  Wave w owns a fixed window of K for the whole launch.
//   * Staging: the activation rows (x, and gamma, beta with LN) become MFMA operand rows in
//     LDS: a per-row power-of-two scale into the fp16 range, a split into 1-3 16-bit terms
//     so that the operand carries >= 22 significant bits, per-group sums for the bias
//     product, and the shifted LayerNorm sums.  When all of K fits (the streaming variant)
//     each wave stages only its own window with its own loads (group reductions by DPP and
//     the gfx950 row swaps) and needs no workgroup barrier for it; long K is staged per
//     chunk by the whole workgroup.  Each wave then keeps its fragments in VGPRs.
//   * Weight stream: lane (c, i) of a wave (c = lane/16, i = lane%16) reads 16 bytes of
//     weight row i per 64-byte step (a dwordx4); 64 lanes cover 16 rows x 64 contiguous
//     bytes per instruction.  Scales and biases of the wave's groups come with one aligned
//     load per lane (even lane groups take biases, odd ones scales; a lane swap pairs them).
//     The next tile's loads are issued before the current tile is computed.
//   * Contraction: v_mfma_f32_16x16x32_{f16,bf16}.  B = 16 weight rows x 32 k of codes fed
//     to the matrix cores as the normal fp16 values 1 + q 2^-bits (the code in the top
//     mantissa bits of 1.0: one shift and one and-or per register), A = up to 16 operand
//     rows x 32 k.  LayerNorm adds the rows gamma and beta, whose products give sum g w and
//     sum b w for the fold.
//   * Per group of 64 codes the MFMA output is a fresh partial P' = G + 2^-bits P, where
//     P = sum q a and G = sum a (the group's operands), and acc += s * P'.  Two more MFMAs
//     per tile take the group sums G as an operand row against the exact fp16 biases and
//     scales: sum_g b G and sum_g s G.  Then s P + b G = 2^bits (s P' - s G) + b G, and the
//     cancellation of s G costs about one bit.
//   * 4-bit rows hold two groups per 64-byte step; after the load, v_permlane32_swap
//     exchanges half-registers between the lane halves so that every MFMA sees one group.
//   * Split-K merge: each wave puts its partial tile into an LDS buffer; the wave that
//     finishes the tile sums the eight partials in wave order.  The streaming variant has no
//     barrier per tile: buffers are handed over with LDS counters (atomics on counters
//     only), so results are bitwise reproducible.
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
// A code q of b bits enters the MFMA as the normal fp16 value 1 + q 2^-b: the code in the
// top b bits of the 10-bit mantissa of 1.0 (0x3C00).  Entered as the subnormal q 2^-24
// instead (the bare bit pattern), the matrix cores lose precision: against exact fp64 dot
// products, a 16x16x32 f16 MFMA of subnormal codes and activations spread over 2^-5..2^15
// was off by up to 2^-14.4 of sum |product|, against 2^-21.9 for the same codes as normal
// values (and no error at all for activations within one binade).
// 4-bit: nibble i of r (bits 4i .. 4i+3) moves to bits 6..9 of a half; halves hold nibbles
// (0, 4), (1, 5), (2, 6), (3, 7).  8-bit: byte i moves to bits 2..9 of a half.
// The normal form has its own cost: the partial carries the offset G, which is removed
// again in fp32, so rows whose operands share a large common part (LayerNorm rows, shifted
// by x[t, 0] and multiplied by gamma ~ 1) lose more than subnormal codes lose.  NC selects
// the normal form (4-bit calls without LayerNorm); otherwise codes enter as subnormals:
// the bit pattern q (q < 1024) is the value q * 2^-24, a mask or a byte permute is the
// whole conversion, and 4-bit high-nibble slots (value 16 q * 2^-24) carry their
// activation divided by 16.
template <int BITS, bool NC>
__device__ __forceinline__ u4_t convert_codes(const u4_t d, int q) {
  u4_t b;
  if constexpr (!NC && BITS == 8) {
    const uint32_t da = d[2 * q], db = d[2 * q + 1];
    b[0] = __builtin_amdgcn_perm(0u, da, 0x0C010C00u);   // bytes 0, 1 -> low byte of each half
    b[1] = __builtin_amdgcn_perm(0u, da, 0x0C030C02u);   // bytes 2, 3
    b[2] = __builtin_amdgcn_perm(0u, db, 0x0C010C00u);
    b[3] = __builtin_amdgcn_perm(0u, db, 0x0C030C02u);
  } else if constexpr (!NC && BITS == 4) {
    const uint32_t r = d[(q & 1) * 2 + (q >> 1)];
    b[0] = r & 0x000F000Fu;
    b[1] = r & 0x00F000F0u;
    b[2] = (r >> 8) & 0x000F000Fu;
    b[3] = (r >> 8) & 0x00F000F0u;
  } else if constexpr (BITS == 8) {
    const uint32_t da = d[2 * q], db = d[2 * q + 1];
    // bytes 0, 1 (2, 3) to the low byte of each half, then two places up under 1.0
    b[0] = (__builtin_amdgcn_perm(0u, da, 0x0C010C00u) << 2) | 0x3C003C00u;
    b[1] = (__builtin_amdgcn_perm(0u, da, 0x0C030C02u) << 2) | 0x3C003C00u;
    b[2] = (__builtin_amdgcn_perm(0u, db, 0x0C010C00u) << 2) | 0x3C003C00u;
    b[3] = (__builtin_amdgcn_perm(0u, db, 0x0C030C02u) << 2) | 0x3C003C00u;
  } else if constexpr (BITS == 4) {
    const uint32_t r = d[(q & 1) * 2 + (q >> 1)];
    b[0] = ((r << 6) & 0x03C003C0u) | 0x3C003C00u;
    b[1] = ((r << 2) & 0x03C003C0u) | 0x3C003C00u;
    b[2] = ((r >> 2) & 0x03C003C0u) | 0x3C003C00u;
    b[3] = ((r >> 6) & 0x03C003C0u) | 0x3C003C00u;
  } else {
    b = d;
  }
  return b;
}
// The unit of a quantized MFMA partial: 2^-bits for normal codes (the partial of a group is
// G + 2^-bits P), 2^-24 for subnormal codes.
template <int BITS, bool NC> __host__ __device__ constexpr float code_mul() {
  return NC ? (BITS == 4 ? 16.0f : 256.0f) : 0x1p24f;
}
// 4-bit subnormal-code operand slots fed by the high nibble of a byte (value 16 q 2^-24)
// carry their activation divided by 16.
template <int BITS, bool NC> __device__ __forceinline__ constexpr bool slot_hi_nibble(int j) {
  return BITS == 4 && !NC && ((j >> 1) & 1) != 0;
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
// Streaming variant: per-wave LN sums S1, S2 of up to 32 rows (each wave sums its window),
// and the merge-buffer handshake words (count, generation, finished, per buffer).
constexpr int kWaveStatFloats = kWaves * 64;
constexpr int kSyncInts = 16;
constexpr int kSyncOffset = (2 * kStatFloats + kExpInts + 2 * kRowMax + kWaveStatFloats) * 4;
constexpr int kHeaderBytes = kSyncOffset + kSyncInts * 4;
// Iterations of a bounded LDS wait (each sleeps ~64 clocks): far longer than any real wait,
// so that a broken handshake ends the kernel instead of hanging the device.
constexpr int kSpinMax = 1 << 22;
// Largest dynamic LDS a launch may ask for (gfx950 has 160 KiB per CU).
// s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima (gfx9 encoding)
constexpr int kWaitVmcnt0 = 0x0F70;
// Elements of an epilogue-input slot: residual rows of up to 32 outputs rows and the constant row, 16 columns.
constexpr int kEpiSlot = 33 * 16;
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

// Reductions over aligned groups of 8 lanes with DPP moves (lane i sees lane i^1, then i^2
// within quads, then the mirrored half of its 8-lane row).  Every lane of a group ends with
// the same value: each step adds two operands that are equal on both partner lanes.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm 1,0,3,2
  v += dpp_f<0x4E>(v);    // quad_perm 2,3,0,1
  v += dpp_f<0x141>(v);   // row_half_mirror
  return v;
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return v;
}
// Operand-row scale exponent for a row maximum amax: 2^e * amax lies in [2^14, 2^15) (e
// clamped to +-126; 0 for a zero or non-finite maximum).
__device__ __forceinline__ int row_exponent(float amax) {
  const uint32_t b = __builtin_bit_cast(uint32_t, amax);
  const int be = (int)(b >> 23) & 0xFF;   // amax >= 0; a subnormal maximum clamps to 126 below
  if (b == 0u || be == 0xFF) return 0;
  const int e = 14 - (be - 127);
  return e > 126 ? 126 : (e < -126 ? -126 : e);
}

// Unpack a 16-byte piece of 8 16-bit elements.
__device__ __forceinline__ void unpack8(const u4_t raw, int dtype, float v[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = elem_to_float((raw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu, dtype);
}

// NS > 0: the streaming variant, where every wave runs exactly NS steps (a window of the row
// that may overlap the previous wave's; the overlapped steps are masked).  NS == 0: the
// chunked variant, up to MAXS steps per wave and chunk.
template <int BITS, bool BF16OP, int MT, int NS = 0, bool NC = false>
struct Fused {
  static constexpr int NM = Fmt<BITS>::kMfma;
  static constexpr int NG = Fmt<BITS>::kGroups > 0 ? Fmt<BITS>::kGroups : 1;
  static constexpr bool QUANT = BITS != 16;
  static constexpr int STEPK = Fmt<BITS>::kStepK;
  static constexpr int MAXS = NS > 0 ? NS : max_steps_for(NM, MT);

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
  // Raw 16-byte pieces of the staged rows (x, gamma, beta) and the gamma piece of each x piece
  // (ones where no LayerNorm multiplies the piece).
  struct StageRegs {
    u4_t raw[kPieceMax], graw[kPieceMax];
  };
  __device__ __forceinline__ static void stage_load(const LinParams& p, int kc0, int kc, int tid, StageRegs& sr) {
    // piece indexing is recomputed at each call (not hoisted out of the chunk loop, where a
    // dozen live addresses would crowd out the fragments)
    asm volatile("" : "+v"(tid));
    const int T = p.T;
    const int srows = T + (p.ln ? 2 : 0);
    const int ppr = kc / 8;                     // pieces per row (a multiple of 8)
    const int total = srows * ppr;
    const uint16_t* x16 = reinterpret_cast<const uint16_t*>(p.x);
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(p.gamma);
    const uint16_t* b16 = reinterpret_cast<const uint16_t*>(p.beta);
    const uint32_t one = p.x_dtype == 1 ? 0x3C003C00u : 0x3F803F80u;
    const uint32_t magic = 0xFFFFFFFFu / (uint32_t)ppr + 1u;   // idx / ppr as a multiply-high
#pragma unroll
    for (int u = 0; u < kPieceMax; ++u) {
      const int idx = tid + kThreads * u;
      sr.graw[u] = (u4_t){one, one, one, one};
      if (idx < total) {
        const int row = (int)__umulhi((uint32_t)idx, magic), pc = idx - row * ppr;
        const bool act = row < T;
        const gptr<const uint16_t> src = pick(act ? x16 : g16, b16, (!act && row != T) ? 1 : 0) +
                                         (act ? (long)row * p.K : 0) + kc0 + 8 * pc;
        sr.raw[u] = *reinterpret_cast<gptr<const u4_t>>(src);
        if (act && p.ln) sr.graw[u] = *reinterpret_cast<gptr<const u4_t>>(pick(g16, g16, 0) + kc0 + 8 * pc);
      }
    }
  }

  // Staging proper.  Pass 1 takes, per source row, the maximum |value| (after the LN shift
  // and gamma) with LDS atomics on the bit patterns (non-negative floats order like their
  // bits), and per 64-wide group the LN partial sums of (x - x[t,0]) and its square.  Pass 2
  // scales each row by 2^e (row_exponent), splits it into terms of the operand type (hi, lo for
  // fp16; hi, mid, lo for bf16) and writes them, in slot order, to the operand rows together
  // with the group sums of each term.  The body is instantiated per input type and for
  // single-term rows, so that no per-element test remains.
  __device__ __forceinline__ static void stage_compute(const LinParams& p, float* stat, int* ex, unsigned* rowmax,
                                                       float* x0s, float* spart, uint16_t* op, float* gsum, int kc0,
                                                       int kc, bool stats, int tid, const StageRegs& sr) {
    asm volatile("" : "+v"(tid));   // as in stage_load
    if (p.x_dtype == 1) {
      if (p.terms == 1) stage_body<1, true>(p, stat, ex, rowmax, x0s, spart, op, gsum, kc0, kc, stats, tid, sr);
      else stage_body<1, false>(p, stat, ex, rowmax, x0s, spart, op, gsum, kc0, kc, stats, tid, sr);
    } else {
      if (p.terms == 1) stage_body<2, true>(p, stat, ex, rowmax, x0s, spart, op, gsum, kc0, kc, stats, tid, sr);
      else stage_body<2, false>(p, stat, ex, rowmax, x0s, spart, op, gsum, kc0, kc, stats, tid, sr);
    }
  }

  template <int XDT>
  __device__ __forceinline__ static void unpack_t(const u4_t raw, float v[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t h = (raw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      v[j] = XDT == 1 ? half_bits_to_float(h) : __builtin_bit_cast(float, h << 16);
    }
  }

  template <int XDT, bool ONE>
  __device__ __forceinline__ static void stage_body(const LinParams& p, float* stat, int* ex, unsigned* rowmax,
                                                    float* x0s, float* spart, uint16_t* op, float* gsum, int kc0,
                                                    int kc, bool stats, int tid, const StageRegs& sr) {
    constexpr int NT = ONE ? 1 : (BF16OP ? 3 : 2);   // terms of an activation row
    const int T = p.T;
    const int srows = T + (p.ln ? 2 : 0);
    const int ppr = kc / 8;
    const int total = srows * ppr;
    const int pitch = op_pitch(kc);
    const int gpr = kc / 64;
    // idx / ppr as a multiply-high: exact while idx * ppr < 2^32
    const uint32_t magic = 0xFFFFFFFFu / (uint32_t)ppr + 1u;
    // the shift x[t, 0] of the LN sums: published by the piece that holds it (the first
    // chunk's), kept in LDS for the later chunks
    if (p.ln && kc0 == 0) {
#pragma unroll
      for (int u = 0; u < kPieceMax; ++u) {
        const int idx = tid + kThreads * u;
        if (kThreads * u < total && idx < total && idx % ppr == 0 && idx / ppr < T)
          x0s[idx / ppr] = XDT == 1 ? half_bits_to_float(sr.raw[u][0] & 0xFFFFu)
                                    : __builtin_bit_cast(float, sr.raw[u][0] << 16);
      }
      lds_barrier();
    }
    // pass 1: row maxima (only rows that are scaled) and LN sums
    if (p.ln || p.scale_act) {
      float x0r1[kPieceMax];
#pragma unroll
      for (int u = 0; u < kPieceMax; ++u) {   // shifts read up front (one LDS round trip)
        const int row = (int)__umulhi((uint32_t)min(tid + kThreads * u, total - 1), magic);
        x0r1[u] = p.ln && row < T ? x0s[row] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kPieceMax; ++u) {
        if (kThreads * u < total) {                    // uniform: some lane of the block is live
          const int idx = tid + kThreads * u;
          const bool live = idx < total;
          const int row = live ? (int)__umulhi((uint32_t)idx, magic) : 0, pc = idx - row * ppr;
          float a[8];
          unpack_t<XDT>(sr.raw[u], a);
          float amax = 0.0f;
          if (p.ln) {
            const bool lnr = row < T;
            const float x0 = x0r1[u];
            float g[8];
            unpack_t<XDT>(sr.graw[u], g);
            float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const float d = a[jj] - x0;
              amax = fmaxf(amax, fabsf(d * g[jj]));
              s1 += d;
              s2 += d * d;
            }
            if (stats) {
              s1 = sum8(s1);
              s2 = sum8(s2);
              if (live && lnr && (pc & 7) == 0) {
                spart[(row * gpr + pc / 8) * 2] = s1;
                spart[(row * gpr + pc / 8) * 2 + 1] = s2;
              }
            }
          } else {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) amax = fmaxf(amax, fabsf(a[jj]));
          }
          amax = max8(amax);
          if (live && (pc & 7) == 0) atomicMax(rowmax + row, __builtin_bit_cast(unsigned, amax));
        }
      }
      lds_barrier();
    }
    // pass 2.  The row maxima (and shifts) of every piece are read up front, from in-range
    // rows also for pieces past the chunk, so that the reads share one LDS round trip.
    uint32_t rmax[kPieceMax];
#pragma unroll
    for (int u = 0; u < kPieceMax; ++u)
      rmax[u] = rowmax[(int)__umulhi((uint32_t)min(tid + kThreads * u, total - 1), magic)];
#pragma unroll
    for (int u = 0; u < kPieceMax; ++u) {
      if (kThreads * u < total) {
        const int idx = tid + kThreads * u;
        const bool live = idx < total;
        const int row = live ? (int)__umulhi((uint32_t)idx, magic) : 0, pc = idx - row * ppr;
        const bool act = row < T;
        const bool need = act ? p.scale_act : p.scale_gb;
        const int e = need ? row_exponent(__builtin_bit_cast(float, rmax[u])) : 0;
        const float scl = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
        const int r0 = act ? NT * row : NT * T + (row - T);
        const int nterm = act ? NT : 1;
        if (live && pc == 0) {
#pragma unroll
          for (int term = 0; term < NT; ++term)
            if (term < nterm) ex[r0 + term] = e;
        }
        float v[8];
        unpack_t<XDT>(sr.raw[u], v);
        if (p.ln) {
          const float x0 = act ? x0s[row] : 0.0f;
          float g[8];
          unpack_t<XDT>(sr.graw[u], g);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) v[jj] = (v[jj] - x0) * g[jj];
        }
        uint32_t el[NT][8];
        float ts[NT];
#pragma unroll
        for (int term = 0; term < NT; ++term) ts[term] = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float sv = v[slot_k<BITS>(jj)] * (slot_hi_nibble<BITS, NC>(jj) ? scl * 0.0625f : scl);
          const uint32_t hi = to_op_bits<BF16OP>(sv);
          el[0][jj] = hi;
          if constexpr (NT >= 2) {
            const float r1 = sv - op_bits_to_float<BF16OP>(hi);
            const uint32_t mid = to_op_bits<BF16OP>(r1);
            el[1][jj] = mid;
            if constexpr (NT == 3) el[2][jj] = to_op_bits<BF16OP>(r1 - op_bits_to_float<BF16OP>(mid));
          }
#pragma unroll
          for (int term = 0; term < NT; ++term)   // group sums of the values as represented, unscaled by 1/16
            ts[term] += op_bits_to_float<BF16OP>(el[term][jj]) * (slot_hi_nibble<BITS, NC>(jj) ? 16.0f : 1.0f);
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
            const float t = sum8(ts[term]);
            if (term < nterm && live && (pc & 7) == 0) gsum[(r0 + term) * gpr + pc / 8] = t;
          }
        }
      } else {
        // pieces past the chunk were loaded on some paths: read them on this one too, or the
        // compiler drains every load in flight before reusing their registers
        asm volatile("" ::"v"(sr.raw[u]), "v"(sr.graw[u]));
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

  // ---- per-wave staging (streaming variant) ------------------------------------------
  // Each wave stages only its own window of K, k0 = s_lo * STEPK .. k0 + WK: the source rows
  // (x rows, then gamma and beta with LN) go through the same transform as above into a
  // block of LDS that only this wave reads.  The power-of-two row scale is per wave (each
  // wave unscales its own partials before the merge), so no value crosses waves before the
  // merge: no atomics and no barrier.  Piece pc = lane + 64 u is source row pc / W8,
  // elements 8 (pc % W8) .. + 7 of the window; W8 <= 64, so the lanes of one row form an
  // aligned group of W8 lanes within one u, and the row reductions are lane butterflies.
  static constexpr int WK = (NS > 0 ? NS : 1) * STEPK;   // window width (elements)
  static constexpr int W8 = WK / 8;                        // pieces per source row
  static constexpr int WG = WK >= 64 ? WK / 64 : 1;        // quantization groups per window
  static constexpr int kWavePieces = 12;                   // pieces per lane, at most
  static_assert(W8 <= 64, "a source row's pieces fit one u");
  __host__ __device__ static constexpr int wave_pitch() { return WK + kRowPad; }
  // Bytes of one wave's block: operand rows, group sums, row exponents.
  __host__ __device__ static constexpr long wave_block_bytes(int rows) {
    return ((long)rows * wave_pitch() * 2 + (long)rows * WG * 4 + (long)rows * 4 + 15) / 16 * 16;
  }
  struct WaveRegs {
    u4_t raw[kWavePieces];    // the piece
    u4_t graw[kWavePieces];   // LN: gamma at the piece's columns
    uint32_t x0[kWavePieces]; // LN: x[row, 0], the shift of the row's sums
  };
  __device__ __forceinline__ static void wave_stage_load(const LinParams& p, int k0, int lane, WaveRegs& wr) {
    const int T = p.T, total = (T + (p.ln ? 2 : 0)) * W8;
    const uint16_t* x16 = reinterpret_cast<const uint16_t*>(p.x);
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(p.gamma);
    const uint16_t* b16 = reinterpret_cast<const uint16_t*>(p.beta);
#pragma unroll
    for (int u = 0; u < kWavePieces; ++u) {
      if (64 * u < total) {   // uniform
        // lanes past the last piece load the last piece again (never written back)
        const int pc = min(lane + 64 * u, total - 1);
        const int row = pc / W8, kp = pc % W8;
        const bool act = row < T;
        const gptr<const uint16_t> src = pick(act ? x16 : g16, b16, (!act && row != T) ? 1 : 0) +
                                         (act ? (long)row * p.K : 0) + k0 + 8 * kp;
        wr.raw[u] = *reinterpret_cast<gptr<const u4_t>>(src);
        if (p.ln) {   // uniform; gamma and x[row, 0] of the piece's (clamped) activation row
          wr.graw[u] = *reinterpret_cast<gptr<const u4_t>>(pick(g16, g16, 0) + k0 + 8 * kp);
          wr.x0[u] = *(pick(x16, x16, 0) + (long)min(row, T - 1) * p.K);
        }
      }
    }
  }
  // Reductions over aligned groups of N lanes (N a power of two <= 64); every lane of a
  // group ends with the group's value.  Within 16-lane rows: DPP moves (xor 1, xor 2, then
  // the mirrored half row and row, which pair every lane with one holding the other half's
  // total); across rows: the gfx950 row swaps, v_permlane16_swap (rows 0<->1, 2<->3) and
  // v_permlane32_swap (lanes l <-> l + 32), which with both operands equal leave one lane of
  // each pair in each result.
  template <int CTRL> __device__ __forceinline__ static uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  }
  template <int N> __device__ __forceinline__ static uint32_t group_max_u(uint32_t v) {
    if constexpr (N >= 2) v = max(v, dpp_u<0xB1>(v));
    if constexpr (N >= 4) v = max(v, dpp_u<0x4E>(v));
    if constexpr (N >= 8) v = max(v, dpp_u<0x141>(v));
    if constexpr (N >= 16) v = max(v, dpp_u<0x140>(v));
    if constexpr (N >= 32) {
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      v = max((uint32_t)r[0], (uint32_t)r[1]);
    }
    if constexpr (N >= 64) {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      v = max((uint32_t)r[0], (uint32_t)r[1]);
    }
    return v;
  }
  template <int N> __device__ __forceinline__ static float group_sum(float v) {
    if constexpr (N >= 2) v += dpp_f<0xB1>(v);
    if constexpr (N >= 4) v += dpp_f<0x4E>(v);
    if constexpr (N >= 8) v += dpp_f<0x141>(v);
    if constexpr (N >= 16) v += dpp_f<0x140>(v);
    if constexpr (N >= 32) {   // both lanes of a pair add the same two values: equal sums
      const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                      false, false);
      v = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
    }
    if constexpr (N >= 64) {
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                      false, false);
      v = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
    }
    return v;
  }
  // s_from: the window's steps before s_from are another wave's (they are staged, but do not
  // count towards this wave's LN sums).
  __device__ __forceinline__ static void wave_stage(const LinParams& p, float* wstat, unsigned char* blk, int lane,
                                                    int s_from, const WaveRegs& wr) {
    asm volatile("" : "+v"(lane));
    if (p.x_dtype == 1) {
      if (p.terms == 1) wave_stage_body<1, true>(p, wstat, blk, lane, s_from, wr);
      else wave_stage_body<1, false>(p, wstat, blk, lane, s_from, wr);
    } else {
      if (p.terms == 1) wave_stage_body<2, true>(p, wstat, blk, lane, s_from, wr);
      else wave_stage_body<2, false>(p, wstat, blk, lane, s_from, wr);
    }
  }
  template <int XDT, bool ONE>
  __device__ __forceinline__ static void wave_stage_body(const LinParams& p, float* wstat, unsigned char* blk,
                                                         int lane, int s_from, const WaveRegs& wr) {
    constexpr int NT = ONE ? 1 : (BF16OP ? 3 : 2);   // terms of an activation row
    const int T = p.T, R = p.rows;
    const int total = (T + (p.ln ? 2 : 0)) * W8;
    uint16_t* op = reinterpret_cast<uint16_t*>(blk);
    float* gsum = reinterpret_cast<float*>(blk + (long)R * wave_pitch() * 2);
    int* ex = reinterpret_cast<int*>(blk + (long)R * wave_pitch() * 2 + (long)R * WG * 4);
#pragma unroll
    for (int u = 0; u < kWavePieces; ++u) {
      if (64 * u < total) {   // uniform: some lane of the wave holds a piece
        const int pc = lane + 64 * u;
        const bool live = pc < total;
        const int row = min(pc, total - 1) / W8, kp = pc % W8;
        const bool act = row < T;
        float v[8];
        unpack_t<XDT>(wr.raw[u], v);
        // LN: activation rows become (x - x[row, 0]) * gamma; gamma and beta rows stay
        if (p.ln) {   // uniform
          const float x0 = act ? (XDT == 1 ? half_bits_to_float(wr.x0[u] & 0xFFFFu)
                                           : __builtin_bit_cast(float, wr.x0[u] << 16)) : 0.0f;
          float g[8];
          unpack_t<XDT>(wr.graw[u], g);
          float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float d = v[jj] - x0;
            s1 += d;
            s2 += d * d;
            v[jj] = act ? d * g[jj] : v[jj];
          }
          if (8 * kp < s_from * STEPK) s1 = s2 = 0.0f;   // another wave's step
          s1 = group_sum<W8>(s1);
          s2 = group_sum<W8>(s2);
          if (live && act && kp == 0) {
            wstat[2 * row] = s1;
            wstat[2 * row + 1] = s2;
          }
        }
        const bool need = act ? p.scale_act : p.scale_gb;
        int e = 0;
        if (p.ln || p.scale_act) {   // uniform; |v| compared as bit patterns (same order)
          uint32_t amax = 0u;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) amax = max(amax, __builtin_bit_cast(uint32_t, v[jj]) & 0x7FFFFFFFu);
          amax = group_max_u<W8>(amax);
          e = need ? row_exponent(__builtin_bit_cast(float, amax)) : 0;
        }
        const float scl = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
        const int r0 = act ? NT * row : NT * T + (row - T);
        const int nterm = act ? NT : 1;
        if (live && kp == 0) {
#pragma unroll
          for (int term = 0; term < NT; ++term)
            if (term < nterm) ex[r0 + term] = e;
        }
        // Terms: hi = the scaled value rounded to the operand type, then the rounded
        // remainders; each remainder is exact before its rounding (one fma).
        uint32_t el[NT][8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float x = v[slot_k<BITS>(jj)];
          const float sj = slot_hi_nibble<BITS, NC>(jj) ? scl * 0.0625f : scl;
          const uint32_t hi = to_op_bits<BF16OP>(x * sj);
          el[0][jj] = hi;
          if constexpr (NT >= 2) {
            const float r1 = fmaf(x, sj, -op_bits_to_float<BF16OP>(hi));
            const uint32_t mid = to_op_bits<BF16OP>(r1);
            el[1][jj] = mid;
            if constexpr (NT == 3) el[2][jj] = to_op_bits<BF16OP>(r1 - op_bits_to_float<BF16OP>(mid));
          }
        }
#pragma unroll
        for (int term = 0; term < NT; ++term) {
          if (term < nterm && live) {
            u4_t w;
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = el[term][2 * r] | (el[term][2 * r + 1] << 16);
            *reinterpret_cast<u4_t*>(op + (long)(r0 + term) * wave_pitch() + 8 * kp) = w;
          }
        }
        if constexpr (QUANT) {
          // Group sum of the row's operand values: scl * sum(v) (a value's terms add up to
          // it within 2^-22 relative; a high-nibble slot's 1/16 operand counts 16 times).
          // It rides on the first term's row; the other terms' rows carry 0.
          float t = 0.0f;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) t += v[jj];
          t = sum8(t) * scl;
          if (live && (kp & 7) == 0) {
#pragma unroll
            for (int term = 0; term < NT; ++term)
              if (term < nterm) gsum[(r0 + term) * WG + kp / 8] = term == 0 ? t : 0.0f;
          }
        }
      } else {
        // pieces past the window were loaded on no path; reading them keeps the compiler's
        // view of every path alike (see compute_core)
        asm volatile("" ::"v"(wr.raw[u]), "v"(wr.graw[u]), "v"(wr.x0[u]));
      }
    }
  }
  // This wave's fragments from its own block (window-relative columns).
  __device__ __forceinline__ void load_frags_wave(const LinParams& p, const unsigned char* blk, int s_from, int c,
                                                  int li) {
    const int R = p.rows;
    const uint16_t* op = reinterpret_cast<const uint16_t*>(blk);
    const float* gsum = reinterpret_cast<const float*>(blk + (long)R * wave_pitch() * 2);
    const int* ex = reinterpret_cast<const int*>(blk + (long)R * wave_pitch() * 2 + (long)R * WG * 4);
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
#pragma unroll
      for (int q = 0; q < NM; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          // rows past R read an in-range row (an A row only feeds its own C row)
          const int r = min(16 * mt + li, R - 1);
          const u4_t v = *reinterpret_cast<const u4_t*>(op + (long)r * wave_pitch() + s * STEPK + frag_base<BITS>(q, c));
          // steps before s_from belong to the previous wave: zero operands, no contribution
          afrag[s][q][mt] = s < s_from ? (u4_t){0u, 0u, 0u, 0u} : v;
        }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = min(16 * mt + 4 * c + v, R - 1);
        unscale[mt][v] = __builtin_bit_cast(float, (uint32_t)(127 - ex[r]) << 23);
      }
      if constexpr (QUANT) {
        const int r = min(16 * mt + li, R - 1);
        uint32_t el[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // groups past the window meet a zero bias, so any finite in-range sum does
          const int gi = min(8 * (c & 1) + j, WG - 1);
          const float v = gsum[r * WG + gi] * (1.0f / (float)(1 << kGsumShift));
          const uint32_t hi = to_op_bits<false>(v);
          const uint32_t lo = to_op_bits<false>(v - op_bits_to_float<false>(hi));
          el[j] = (c >> 1) ? lo : hi;
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) gfrag[mt][w] = el[2 * w] | (el[2 * w + 1] << 16);
      }
    }
  }

  // ---- per-wave fragment load from the staged rows ----------------------------------
  __device__ __forceinline__ void load_frags(const LinParams& p, const int* ex, const uint16_t* op, const float* gsum,
                                             int kc0, int kc, int cs0, int s_lo, int s_from, int c, int li) {
    const int R = p.rows, pitch = op_pitch(kc), gpr = kc / 64;
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
#pragma unroll
      for (int q = 0; q < NM; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          // Rows past R and steps past the slice read in-range data that is never used: an
          // A row only feeds its own C row, and steps >= nsw are skipped.  No branches, so
          // all reads share one LDS round trip.
          const int r = min(16 * mt + li, R - 1);
          const int kk = min((s_lo + s) * STEPK + frag_base<BITS>(q, c) - kc0, kc - 8);
          afrag[s][q][mt] = *reinterpret_cast<const u4_t*>(op + (long)r * pitch + max(kk, 0));
        }
    if constexpr (NS > 0) {
      // steps before s_from belong to the previous wave: zero operands, no contribution
#pragma unroll
      for (int s = 0; s < MAXS; ++s)
#pragma unroll
        for (int q = 0; q < NM; ++q)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (s < s_from) afrag[s][q][mt] = (u4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {   // 2^-e; rows past R: any finite factor (never read back)
        const int r = min(16 * mt + 4 * c + v, R - 1);
        unscale[mt][v] = __builtin_bit_cast(float, (uint32_t)(127 - ex[r]) << 23);
      }
      if constexpr (QUANT) {
        const int r = 16 * mt + li;
        uint32_t el[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // slots past the slice meet a zero bias (compute_tile), so any finite
          // in-range group sum does
          const int gi = 8 * (c & 1) + j;
          const int gl = min((s_lo - cs0) * NG + gi, gpr - 1);
          const float v = gsum[min(r, R - 1) * gpr + gl] * (1.0f / (float)(1 << kGsumShift));
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

  // Epilogue inputs of a linear tile: residual[t, n0 .. n0+15] for t < T and constant[n0 ..
  // n0+15] (n0 = 16 tile), fetched by the workgroup a tile ahead, one element per thread and
  // round (consecutive lanes, consecutive columns), into an LDS slot [T + 1][16] of the
  // input type.  Nothing is loaded when the call has neither.
  struct EpRegs {
    uint32_t v[2];   // (T + 1) * 16 <= 528 elements: at most two per thread
  };
  __device__ __forceinline__ static void ep_issue(const LinParams& p, int tile, int tid, EpRegs& e) {
    e.v[0] = e.v[1] = 0u;
    if (p.gateup || !(p.res || p.add)) return;   // uniform
    const gptr<const uint16_t> z16 = pick(reinterpret_cast<const uint16_t*>(g_zero16),
                                          reinterpret_cast<const uint16_t*>(g_zero16), 0);
    const gptr<const uint16_t> rp = pick(reinterpret_cast<const uint16_t*>(p.res), reinterpret_cast<const uint16_t*>(p.res), 0);
    const gptr<const uint16_t> ap = pick(reinterpret_cast<const uint16_t*>(p.add), reinterpret_cast<const uint16_t*>(p.add), 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int el = tid + kThreads * i, row = el >> 4, n = tile * 16 + (el & 15);
      const bool ok = tile < p.ntiles && n < p.N && row <= p.T;
      const bool isres = row < p.T;
      const bool have = ok && (isres ? p.res != nullptr : p.add != nullptr);
      e.v[i] = *(have ? (isres ? rp + (long)row * p.N + n : ap + n) : z16);
    }
  }
  __device__ __forceinline__ static void ep_commit(const LinParams& p, int tid, const EpRegs& e, uint16_t* slot) {
    asm volatile("" ::"v"(e.v[0]), "v"(e.v[1]));   // read on every path (see compute_core)
    if (p.gateup || !(p.res || p.add)) return;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int el = tid + kThreads * i;
      if (el < (p.T + 1) * 16) slot[el] = (uint16_t)e.v[i];
    }
  }

  // Issue the loads of a tile's codes, scales and biases for steps [s_lo, s_lo + nsw).
  // One base address per lane and tile, then immediate offsets per step.  A lane with no
  // row (n >= N, or a tile past the last) streams from the zero buffer instead, so every
  // tile issues the same loads; steps >= nsw (uniform) are skipped.  Rows must consist of
  // whole 64-byte steps (4-bit K = 64 mod 128 goes through the chunked variant).
  template <bool CHECKED = false, bool SB = true>
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
      const gptr<const char> a = (NS > 0 || s < nsw) ? cb + s * 64 : zero + 16 * c;
      if constexpr (CHECKED) {   // a row may end half-way through its last step
        const bool in = (long)(s_lo + s) * 64 + 16 * c < row_bytes;
        r.dw[s] = *reinterpret_cast<gptr<const u4_t>>(in ? a : zero + 16 * c);
      } else {
        r.dw[s] = *reinterpret_cast<gptr<const u4_t>>(a);
      }
    }
    if constexpr (QUANT && SB) {
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

  // One tile through the fragments: codes dw, per-step scale words sc (the step's NG fp16
  // scales, group g in bits 16g) and the bias operand bfr (slot j of lane group c holds the
  // bias of this wave's group 8*(c&1) + j, 0 past the slice).
  __device__ __forceinline__ void compute_core(int nsw, const u4_t dw[MAXS], const uint32_t sc[MAXS], const u4_t& bfr,
                                               const u4_t& sfr, f4_t acc[MT]) {
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      if (NS > 0 || s < nsw) {   // streaming: every step runs (masked steps have zero operands)
        u4_t d = dw[s];
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
              const u4_t b = convert_codes<BITS, NC>(d, q);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) cg[g][mt] = mfma<BF16OP>(afrag[s][q][mt], b, cg[g][mt]);
            }
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const float sf = half_bits_to_float((sc[s] >> (16 * g)) & 0xFFFFu);
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
        asm volatile("" ::"v"(dw[s]), "v"(sc[s]));
      }
    }
    if constexpr (QUANT) {
      // sum_g b[n, g] G_g (G_g: group g's operand sum, held times 2^-kGsumShift), and for
      // normal codes sum_g s[n, g] G_g: acc = sum s P' - sum s G + 2^-bits sum b G, in units
      // of 2^-bits (subnormal codes: acc = sum s P + 2^-24 sum b G, in units of 2^-24)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (NC) {
          const f4_t cs = mfma<false>(gfrag[mt], sfr, (f4_t){0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[mt][v] = fmaf(cs[v], -(float)(1 << kGsumShift), acc[mt][v]);
        }
        const f4_t cb = mfma<false>(gfrag[mt], bfr, (f4_t){0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[mt][v] = fmaf(cb[v], (float)(1 << kGsumShift) / code_mul<BITS, NC>(), acc[mt][v]);
      }
    }
  }

  // A tile whose scales and biases came with its codes (chunked variant).
  __device__ __forceinline__ void compute_tile(int nsw, int c, const TileRegs& r, f4_t acc[MT]) {
    u4_t bfr = (u4_t){0u, 0u, 0u, 0u}, sfr = (u4_t){0u, 0u, 0u, 0u};
    if constexpr (QUANT) {
      // slot j of lane group c: group 8 (c & 1) + j's bias (scale); groups past this wave's
      // slice get 0 (their loads were skipped)
      auto operand = [&](const uint32_t (&v)[MAXS], u4_t& out) __attribute__((always_inline)) {
        uint32_t el[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t lo = (j < MAXS * NG && j < nsw * NG) ? (v[j / NG] >> (16 * (j % NG))) & 0xFFFFu : 0u;
          const uint32_t hi = (8 + j < MAXS * NG && 8 + j < nsw * NG)
                                  ? (v[(8 + j) / NG] >> (16 * ((8 + j) % NG))) & 0xFFFFu : 0u;
          el[j] = (c & 1) ? hi : lo;
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = el[2 * w] | (el[2 * w + 1] << 16);
      };
      operand(r.bi, bfr);
      if constexpr (NC) operand(r.sc, sfr);
    }
    compute_core(nsw, r.dw, r.sc, bfr, sfr, acc);
  }

  // ---- per-wave scales and biases (streaming variant) --------------------------------
  // Each wave loads the scales and biases of its own window for a tile's 16 rows with one
  // load per lane: lanes of even lane groups c take row li's biases, odd ones its scales
  // (WGR fp16 values, one aligned load: K is a multiple of 512 and the window starts at a
  // multiple of NS steps), and v_permlane16_swap hands each lane its partner group's half.
  static constexpr int WGR = NS * NG;                    // groups of a window
  static constexpr int WD = WGR >= 2 ? WGR / 2 : 1;      // dwords they take
  struct SbW {
    u4_t v;
  };
  __device__ __forceinline__ static void sbw_issue(const LinParams& p, int tile, int s_lo, int c, int li, SbW& r) {
    r.v = (u4_t){0u, 0u, 0u, 0u};
    if constexpr (QUANT) {
      int proj, n;
      tile_row(p, tile, li, proj, n);
      const bool valid = tile < p.ntiles && n < p.N;
      const int G = p.K / 64;
      const gptr<const uint16_t> base = pick((c & 1) ? p.sc[0] : p.bi[0], (c & 1) ? p.sc[1] : p.bi[1], proj);
      const gptr<const uint16_t> zh = pick(reinterpret_cast<const uint16_t*>(g_zero16),
                                           reinterpret_cast<const uint16_t*>(g_zero16), 0);
      const gptr<const uint16_t> src = valid ? base + (long)n * G + (long)s_lo * NG : zh;
      if constexpr (WGR == 1) {
        r.v[0] = *src;
      } else if constexpr (WGR == 2) {
        r.v[0] = *reinterpret_cast<gptr<const uint32_t>>(src);
      } else if constexpr (WGR == 4) {
        typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
        const u2_t d = *reinterpret_cast<gptr<const u2_t>>(src);
        r.v[0] = d[0];
        r.v[1] = d[1];
      } else {
        static_assert(WGR == 8, "windows of 1, 2, 4 or 8 groups");
        r.v = *reinterpret_cast<gptr<const u4_t>>(src);
      }
    }
  }
  // A tile from the code registers and this wave's scale/bias registers.
  __device__ __forceinline__ void compute_regs(int s_from, int c, const SbW& sb, const u4_t dw[MAXS], f4_t acc[MT]) {
    static_assert(NS > 0, "the streaming variant");
    uint32_t sc[MAXS];
    u4_t bfr = (u4_t){0u, 0u, 0u, 0u}, sfr = (u4_t){0u, 0u, 0u, 0u};
    if constexpr (QUANT) {
      uint32_t scl[WD], bia[WD];
#pragma unroll
      for (int j = 0; j < WD; ++j) {
        // with both operands equal, result 0 holds rows 0, 0, 2, 2 and result 1 rows 1, 1, 3, 3
        const auto r = __builtin_amdgcn_permlane16_swap(sb.v[j], sb.v[j], false, false);
        const uint32_t own = (c & 1) ? (uint32_t)r[1] : (uint32_t)r[0];
        const uint32_t partner = (c & 1) ? (uint32_t)r[0] : (uint32_t)r[1];
        scl[j] = (c & 1) ? own : partner;
        bia[j] = (c & 1) ? 0u : own;   // odd lane groups feed the bias MFMA groups 8..15: none
      }
#pragma unroll
      for (int s = 0; s < MAXS; ++s) {
        const uint32_t v = NG == 2 ? scl[s] : (scl[s >> 1] >> (16 * (s & 1))) & 0xFFFFu;
        sc[s] = s >= s_from ? v : 0u;   // steps before s_from are another wave's
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int g0 = 2 * w, g1 = 2 * w + 1;
        const uint32_t v = w < WD ? bia[w < WD ? w : 0] : 0u;
        // the scale operand: even lane groups hold groups 0..7, odd ones groups 8..15 (none)
        const uint32_t u = (w < WD && !(c & 1)) ? scl[w < WD ? w : 0] : 0u;
        const bool ok0 = g0 < WGR && g0 >= s_from * NG, ok1 = g1 < WGR && g1 >= s_from * NG;
        bfr[w] = (ok0 ? (v & 0xFFFFu) : 0u) | (ok1 ? (v & 0xFFFF0000u) : 0u);
        sfr[w] = (ok0 ? (u & 0xFFFFu) : 0u) | (ok1 ? (u & 0xFFFF0000u) : 0u);
      }
    } else {
#pragma unroll
      for (int s = 0; s < MAXS; ++s) sc[s] = 0u;
    }
    compute_core(NS, dw, sc, bfr, sfr, acc);
  }

  // Epilogue inputs of the outputs a finishing lane owns (linear with residual or constant):
  // residual[t, n] for its NO rows and constant[n], loaded a tile ahead.  Every wave issues
  // the loads, from the zero buffer where it does not finish the tile's block b (< MT):
  // a load on one path only would make the compiler copy, and so wait for, its value.
  struct EpW {
    uint32_t v[5];
  };
  // nt: operand terms per activation row (1 or 2): the lane owns 4 / nt output rows.
  __device__ __forceinline__ static void epw_issue(const LinParams& p, int tile, int b, int nt, int c, int li, EpW& e) {
    const gptr<const uint16_t> z16 = pick(reinterpret_cast<const uint16_t*>(g_zero16),
                                          reinterpret_cast<const uint16_t*>(g_zero16), 0);
    const gptr<const uint16_t> rp = pick(reinterpret_cast<const uint16_t*>(p.res), reinterpret_cast<const uint16_t*>(p.res), 0);
    const gptr<const uint16_t> ap = pick(reinterpret_cast<const uint16_t*>(p.add), reinterpret_cast<const uint16_t*>(p.add), 0);
    const int n = tile * 16 + li;
    const bool nok = b < MT && tile < p.ntiles && n < p.N;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      const int t = ((16 * b + 4 * c) >> (nt - 1)) + o;
      // 32 x 32 -> 64-bit offset in one multiply-add (a 64-bit product would read an
      // undefined high half, which may be a register still waiting for a load)
      const uint64_t off = (uint64_t)(uint32_t)t * (uint32_t)p.N + (uint32_t)n;
      e.v[o] = *((p.res && nok && o < (4 >> (nt - 1)) && t < p.T) ? rp + off : z16);
    }
    e.v[4] = *((p.add && nok) ? ap + n : z16);
  }
};

// Per-row LN moments from the shifted sums S1, S2 of row t: m = S1 / K (the mean of the
// shifted row), var = S2 / K - m^2 (biased, clamped at 0), rstd = 1 / sqrt(var + eps).
__device__ __forceinline__ void row_moments(const LinParams& p, const float* stat, float* mr, int t) {
  const float m = stat[2 * t] / (float)p.K;
  const float var = fmaxf(stat[2 * t + 1] / (float)p.K - m * m, 0.0f);
  mr[2 * t] = m;
  mr[2 * t + 1] = 1.0f / sqrtf(var + p.eps);
}

// Partial of C row r, column col written by wave w for a tile (double buffer buf).
template <int MT>
__device__ __forceinline__ float partial_at(const float* red, int buf, int w, int r, int col) {
  return red[((buf * kWaves + w) * MT + (r >> 4)) * 256 + (16 * ((r & 15) >> 2) + col) * 4 + (r & 3)];
}

// Merge, LN fold, epilogue and store of one tile, spread over all lanes of the workgroup:
// each output takes 8 consecutive lanes, lane w reading wave w's partials (all reads are
// issued before any arithmetic, at in-range rows), and the 8 are summed with a fixed DPP
// tree.  A gate/up output pairs the 8 lanes of g with the next 8 lanes holding u.  The
// storing lane is the group's first.  Epilogue order as [p1] `_linear_kernel`: GELU, then
// residual, then constant; one rounding to the output type.
template <int MT, int NT>
__device__ __forceinline__ void finalize(const LinParams& p, const float* red, const float* mr, const uint16_t* epi,
                                         int buf, int tile, int tid) {
  const int lane = tid & 63, wv = tid >> 6, w = lane & 7;
  const int terms = p.terms, T = p.T;
  const int rounds = (T + 3) >> 2;   // 64 linear (32 gate/up) outputs per round
  for (int rd = 0; rd < rounds; ++rd) {
    int t, col, n, half;
    if (p.gateup) {
      const int o = rd * 32 + wv * 4 + (lane >> 4);
      t = o >> 3; half = (lane >> 3) & 1; col = (o & 7) + 8 * half; n = tile * 8 + (o & 7);
    } else {
      const int o = rd * 64 + wv * 8 + (lane >> 3);
      t = o >> 4; half = 0; col = o & 15; n = tile * 16 + col;
    }
    const bool valid = t < T && n < p.N;
    const int tc = min(t, T - 1);
    float part[NT];
#pragma unroll
    for (int term = 0; term < NT; ++term) part[term] = partial_at<MT>(red, buf, w, term < terms ? terms * tc + term : 0, col);
    const float gv = partial_at<MT>(red, buf, w, p.ln ? terms * T : 0, col);
    const float bv = partial_at<MT>(red, buf, w, p.ln ? terms * T + 1 : 0, col);
    const float m = mr[2 * tc], rstd = mr[2 * tc + 1];
    const uint32_t rb = epi[tc * 16 + (col & 15)], ab = epi[T * 16 + (col & 15)];
    float P = 0.0f;
#pragma unroll
    for (int term = 0; term < NT; ++term) P += term < terms ? part[term] : 0.0f;
    P = sum8(P);
    float v = P;
    if (p.ln) v = rstd * (P - m * sum8(gv)) + sum8(bv);   // uniform
    if (p.gateup) {
      // u from the next 8 lanes (rotate by 8 within the 16-lane row); silu(g) * u with the
      // hardware exp2 and reciprocal (a few ulp; far inside the tolerance)
      const float u = dpp_f<0x128>(v);   // row_ror:8
      v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;
    } else {
      if (p.act == 1) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
      if (p.res) v += elem_to_float(rb, p.x_dtype);
      if (p.add) v += elem_to_float(ab, p.x_dtype);
    }
    if (valid && w == 0 && half == 0) store_out(p.y, p.y_dtype, (long)t * p.N + n, v);
  }
}

// Merge, LN fold, epilogue and store of 16-row block b of a tile, by one wave.  Each lane
// sums the eight waves' partials of its own C position (16-byte LDS reads where the
// partials were written: no bank conflicts) in wave order, then finishes the outputs of its
// rows in registers: rows NT t .. NT t + NT - 1 of an activation row t lie in one lane
// (NT = 1 or 2).  With LN, G_n and B_n (the gamma and beta rows) are merged from the
// partials as well.  A gate/up tile pairs column n (gate) with column n + 8 (up) of the same
// 16-lane row.  part: the tile's partials, [wave][MT][256].  res / add: the lane's residual
// values (one per output row) and constant.  Epilogue order as [p1] `_linear_kernel`: GELU,
// then residual, then constant; one rounding to the output type.
// bad: the tile's merge wait gave up; its outputs are stored as NaN (a select, not a branch,
// so that the stores and their wait counts are the same on both paths).
template <int MT, int NT>
__device__ __forceinline__ void finalize_block(const LinParams& p, const float* part, const float* mr, int b, int tile,
                                               int lane, const float res[4 / NT], float add, bool bad = false) {
  const int c = lane >> 4, li = lane & 15;
  const int T = p.T;
  // all eight reads in flight before the first add (one LDS round trip)
  f4_t pv[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) pv[w] = *reinterpret_cast<const f4_t*>(part + (w * MT + b) * 256 + lane * 4);
  __builtin_amdgcn_sched_barrier(0);
  f4_t m = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] += pv[w][j];
  float G = 0.0f, B = 0.0f;
  if (p.ln) {   // uniform: G_n, B_n from rows NT T and NT T + 1, column li
    const int rg = NT * T, rb = rg + 1;
    const float* pg = part + (rg >> 4) * 256 + ((((rg & 15) >> 2) << 4) | li) * 4 + (rg & 3);
    const float* pb = part + (rb >> 4) * 256 + ((((rb & 15) >> 2) << 4) | li) * 4 + (rb & 3);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      G += pg[w * MT * 256];
      B += pb[w * MT * 256];
    }
  }
  constexpr int NO = 4 / NT;   // activation rows per lane
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    const int t = (16 * b + 4 * c) / NT + o;
    const int tc = min(t, T - 1);
    float v = 0.0f;
#pragma unroll
    for (int term = 0; term < NT; ++term) v += m[o * NT + term];
    if (p.ln) v = mr[2 * tc + 1] * (v - mr[2 * tc] * G) + B;
    if (p.gateup) {
      // u from the lane 8 to the right in the 16-lane row; silu(g) * u with the hardware
      // exp2 and reciprocal (a few ulp; far inside the tolerance)
      const float u = dpp_f<0x128>(v);   // row_ror:8
      v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;
      const int n = tile * 8 + li;
      if (t < T && li < 8 && n < p.N) store_out(p.y, p.y_dtype, (long)t * p.N + n, bad ? __builtin_nanf("") : v);
    } else {
      if (p.act == 1) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
      if (p.res) v += res[o];
      if (p.add) v += add;
      const int n = tile * 16 + li;
      if (t < T && n < p.N) store_out(p.y, p.y_dtype, (long)t * p.N + n, bad ? __builtin_nanf("") : v);
    }
  }
}

// A tile whose partials sit in double-buffer half buf, finished by the waves that own its
// blocks: wave w takes block b = (w - rot) mod 8 (when b < MT), rot counting the
// workgroup's tiles, so that the work rotates over the waves.  Epilogue inputs come from
// the LDS slot epi ([T + 1][16] of the input type).
template <int MT, int NT>
__device__ __forceinline__ void finalize_rows(const LinParams& p, const float* red, const float* mr, const uint16_t* epi,
                                              int buf, int tile, int rot, int wv, int lane) {
  const int c = lane >> 4, li = lane & 15;
  for (int b = (wv - rot) & 7; b < MT; b += kWaves) {   // uniform per wave
    float res[4 / NT];
#pragma unroll
    for (int o = 0; o < 4 / NT; ++o) {
      const int t = min((16 * b + 4 * c) / NT + o, p.T - 1);
      res[o] = p.res ? elem_to_float(epi[t * 16 + li], p.x_dtype) : 0.0f;
    }
    const float add = p.add ? elem_to_float(epi[p.T * 16 + li], p.x_dtype) : 0.0f;
    finalize_block<MT, NT>(p, red + buf * kWaves * MT * 256, mr, b, tile, lane, res, add);
  }
}

// The whole tile by one wave, for rows of three terms (they straddle lanes and blocks):
// the lanes merge every block into wave 0's partials (in place, each lane its own
// positions), then lane (q, n) finishes outputs (4 i + q, n) from the merged rows.  The
// residual and constant are read from global memory here (a rare path).
template <int MT>
__device__ __forceinline__ void finalize_tile3(const LinParams& p, float* part, const float* mr, int tile, int lane,
                                               bool bad = false) {
  constexpr int NT = 3;
  const int T = p.T;
#pragma unroll
  for (int b = 0; b < MT; ++b) {
    f4_t m = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f4_t v = *reinterpret_cast<const f4_t*>(part + (w * MT + b) * 256 + lane * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) m[j] += v[j];
    }
    *reinterpret_cast<f4_t*>(part + b * 256 + lane * 4) = m;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  auto row = [&](int r, int n) __attribute__((always_inline)) {
    return part[(r >> 4) * 256 + ((((r & 15) >> 2) << 4) | n) * 4 + (r & 3)];
  };
  const int q = lane >> 4, col = lane & 15;
  const float G = p.ln ? row(NT * T, col) : 0.0f, B = p.ln ? row(NT * T + 1, col) : 0.0f;
  for (int t0 = 0; t0 < T; t0 += 4) {
    const int t = t0 + q, tc = min(t, T - 1);
    float v = row(NT * tc, col) + row(NT * tc + 1, col) + row(NT * tc + 2, col);
    if (p.ln) v = mr[2 * tc + 1] * (v - mr[2 * tc] * G) + B;
    if (p.gateup) {
      const float u = dpp_f<0x128>(v);   // row_ror:8
      v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;
      const int n = tile * 8 + col;
      if (t < T && col < 8 && n < p.N) store_out(p.y, p.y_dtype, (long)t * p.N + n, bad ? __builtin_nanf("") : v);
    } else {
      const int n = tile * 16 + col;
      const bool ok = t < T && n < p.N;
      if (p.act == 1) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
      if (p.res && ok) v += elem_to_float(reinterpret_cast<const uint16_t*>(p.res)[(long)t * p.N + n], p.x_dtype);
      if (p.add && ok) v += elem_to_float(reinterpret_cast<const uint16_t*>(p.add)[n], p.x_dtype);
      if (ok) store_out(p.y, p.y_dtype, (long)t * p.N + n, bad ? __builtin_nanf("") : v);
    }
  }
}

// Bounded wait until an LDS word equals v (all lanes read the same word): at most `limit`
// polls.  Returns whether the word reached v (uniform over the wave); a wait that gives up
// is reported by the caller (device counter, NaN outputs), never ignored.
__device__ __forceinline__ bool lds_wait_eq(const int* a, int v, int limit) {
#pragma nounroll
  for (int it = 0; it < limit; ++it) {
    const int cur = __builtin_amdgcn_readfirstlane(__hip_atomic_load(a, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (cur == v) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// EPI (streaming variant): the call is a linear with residual or constant inputs.
template <int BITS, bool BF16OP, int MT, bool CHUNKED, int NS, bool EPI, bool NC>
__global__ __launch_bounds__(kThreads) void fused_kernel(const LinParams p) {
  static_assert(CHUNKED == (NS == 0), "the streaming variant has a fixed step count");
  static_assert(!NC || BITS == 4, "normal codes: 4-bit weights");
  static_assert(!(CHUNKED && EPI), "the chunked variant stages epilogue inputs in LDS");
  using S = Fused<BITS, BF16OP, MT, NS, NC>;
  constexpr int STEPK = S::STEPK;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  float* stat = reinterpret_cast<float*>(lds_raw);
  int* ex = reinterpret_cast<int*>(lds_raw + kStatFloats * 4);
  unsigned* rowmax = reinterpret_cast<unsigned*>(lds_raw + (kStatFloats + kExpInts) * 4);
  float* x0s = reinterpret_cast<float*>(lds_raw + (kStatFloats + kExpInts + kRowMax) * 4);
  float* mr = reinterpret_cast<float*>(lds_raw + (kStatFloats + kExpInts + 2 * kRowMax) * 4);
  float* wstat = reinterpret_cast<float*>(lds_raw + (2 * kStatFloats + kExpInts + 2 * kRowMax) * 4);
  unsigned char* region = lds_raw + kHeaderBytes;
  float* red = reinterpret_cast<float*>(region);

  const int tid = threadIdx.x, lane = tid & 63, c = lane >> 4, li = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  // This wave's steps of chunk ch: [s_lo, s_lo + nsw), of which those before s_from are
  // another wave's.  Chunked: an even split of the chunk (s_from = 0).  Streaming: a window
  // of NS steps that starts at wv * NS, moved back to end at the row's last step when it
  // would run past it (NS <= steps), so that every load stays inside the row.
  auto slice = [&](int ch, int& cs0, int& s_lo, int& nsw, int& s_from) __attribute__((always_inline)) {
    if constexpr (NS > 0) {
      cs0 = 0;
      s_lo = min(wv * NS, p.steps - NS);
      s_from = wv * NS - s_lo;
      nsw = NS;
    } else {
      cs0 = ch * p.chunk_steps;
      const int sc = min(p.chunk_steps, p.steps - cs0);
      s_lo = cs0 + (wv * sc) / kWaves;
      nsw = cs0 + ((wv + 1) * sc) / kWaves - s_lo;
      s_from = 0;
    }
  };
  // Stage chunk ch into LDS and load this wave's fragments from it.
  S st;
  // Stage chunk ch (its pieces already in sr), run after_stage, load this wave's fragments.
  auto prepare = [&](int ch, bool stats, int& cs0, int& s_lo, int& nsw, int& s_from, const typename S::StageRegs& sr,
                     auto&& after_stage) __attribute__((always_inline)) {
    slice(ch, cs0, s_lo, nsw, s_from);
    const int kc0 = cs0 * STEPK;
    const int kc = min(p.chunk_steps * STEPK, p.K - kc0);
    uint16_t* op = reinterpret_cast<uint16_t*>(region);
    float* gsum = reinterpret_cast<float*>(region + (long)p.rows * op_pitch(kc) * 2);
    float* spart = gsum + (long)p.rows * (kc / 64);
    if (tid < kRowMax) rowmax[tid] = 0u;
    lds_barrier();
    S::stage_compute(p, stat, ex, rowmax, x0s, spart, op, gsum, kc0, kc, stats, tid, sr);
    after_stage();
    lds_barrier();
    if (stats && p.ln && tid < p.T) row_moments(p, stat, mr, tid);   // read after a later barrier
    st.load_frags(p, ex, op, gsum, kc0, kc, cs0, s_lo, s_from, c, li);
    lds_barrier();
  };
  // This wave's partials of a tile into LDS (double-buffered by tile parity).
  auto write_partials = [&](const f4_t acc[MT], int buf, float* base) __attribute__((always_inline)) {
    float* rb = base + (buf * kWaves + wv) * MT * 256;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f4_t v;
#pragma unroll
      for (int j = 0; j < 4; ++j)   // quantized partials are in units of 2^-bits (code_mul)
        v[j] = (S::QUANT ? acc[mt][j] * code_mul<BITS, NC>() : acc[mt][j]) * st.unscale[mt][j];
      *reinterpret_cast<f4_t*>(rb + mt * 256 + lane * 4) = v;
    }
  };
  // Merge the waves' partials of a tile and finish it (epilogue inputs from slot `epi`).
  // Finish a tile whose partials sit in buffer buf (rot: the tile's index among this
  // workgroup's tiles; a barrier must separate the partial writes from this).
  auto fin = [&](int tile, int rot, int buf, const uint16_t* epi) __attribute__((always_inline)) {
    if (BF16OP && p.terms == 3) finalize<MT, 3>(p, red, mr, epi, buf, tile, tid);   // rows straddle lanes
    else if (p.terms == 1) finalize_rows<MT, 1>(p, red, mr, epi, buf, tile, rot, wv, lane);
    else finalize_rows<MT, 2>(p, red, mr, epi, buf, tile, rot, wv, lane);
  };
  auto finish = [&](int tile, int rot, int buf, const uint16_t* epi) __attribute__((always_inline)) {
    lds_barrier();
    fin(tile, rot, buf, epi);
  };

  if (tid < kStatFloats) stat[tid] = 0.0f;
  int cs0, s_lo, nsw, s_from;
  if constexpr (!CHUNKED) {
    // All of K fits: build the fragments once, then stream tiles with the next tile's codes,
    // scales and biases always in flight (two register sets alternate: a copy at the end of
    // an iteration would make the compiler wait for the prefetch).  The waves do not meet at
    // a barrier per tile: each streams its own window, and the partials of a tile meet in
    // one of NB LDS buffers through a handshake of three words per buffer:
    //   gen  the tile the buffer is open for; a wave writes its partials only once it is;
    //   cnt  waves whose partials are in; the finishing waves wait for all eight;
    //   fin  finishing waves done; the last one empties the buffer and opens it for tile + NB.
    // Every wait is for earlier work of tiles in order, so no wait can close a cycle, and
    // each is bounded besides.
    constexpr int NB = MT <= 2 ? 4 : 2;   // merge buffers in flight
    slice(0, cs0, s_lo, nsw, s_from);
    int tile = blockIdx.x;
    unsigned char* blk = region + wv * S::wave_block_bytes(p.rows);
    int* pcnt = reinterpret_cast<int*>(lds_raw + kSyncOffset);
    int* pgen = pcnt + NB;
    int* pfin = pgen + NB;
    const bool three = BF16OP && p.terms == 3;   // rows straddle lanes: one wave finishes a tile
    const int nfin = three ? 1 : MT;               // finishing waves per tile
    // Issue order: this wave's window of the activation rows, then the first tile's scales
    // and codes, so that staging waits for its own rows only (loads complete in order) and
    // the weight stream runs under it.
    typename S::WaveRegs wr;
    S::wave_stage_load(p, s_lo * STEPK, lane, wr);
    typename S::SbW sa, sb;
    S::sbw_issue(p, tile, s_lo, c, li, sa);
    typename S::TileRegs ra, rb;
    S::template load_tile<false, false>(p, tile, s_lo, nsw, c, li, ra);
    S::wave_stage(p, wstat + wv * 64, blk, lane, s_from, wr);
    // the block is this wave's own: its writes only need to have completed
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    st.load_frags_wave(p, blk, s_from, c, li);
    if (tid < NB) {
      pcnt[tid] = 0;
      pfin[tid] = 0;
      pgen[tid] = tid;
    }
    // every wave is done with its block before the merge partials reuse the region; the LN
    // sums and the handshake words are visible to all
    lds_barrier();
    if (p.ln) {   // uniform: LN moments from the waves' sums, for every finishing wave
      if (tid < p.T) {
        float s1 = 0.0f, s2 = 0.0f;
        for (int w = 0; w < kWaves; ++w) { s1 += wstat[w * 64 + 2 * tid]; s2 += wstat[w * 64 + 2 * tid + 1]; }
        const float m = s1 / (float)p.K;
        const float var = fmaxf(s2 / (float)p.K - m * m, 0.0f);
        mr[2 * tid] = m;
        mr[2 * tid + 1] = 1.0f / sqrtf(var + p.eps);
      }
      lds_barrier();
    }
    const int G = gridDim.x;
    // block of tile rot this wave finishes (none when >= nfin)
    auto my_block = [&](int rot) __attribute__((always_inline)) { return (wv - rot) & 7; };
    // Put this wave's partials of tile rot into its buffer once the buffer is open for it.
    // Give-ups of the bounded waits are counted in a register and added to p.timeouts once,
    // at the end of the kernel (a global atomic inside a branch here would make the compiler
    // wait for every load in flight at the join).  A put writes after its wait either way, so
    // that no branch separates the compute from the next tile; a finishing wave that gives up
    // stores NaN.  Any give-up is therefore reported, by the counter and/or NaN outputs.
    int gave_up = 0;
    auto put = [&](const f4_t acc[MT], int rot) __attribute__((always_inline)) {
      const int q = rot & (NB - 1);
      gave_up += lds_wait_eq(pgen + q, rot, p.spin) ? 0 : 1;
      write_partials(acc, 0, red + q * kWaves * MT * 256);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");   // the writes are done
      if (lane == 0) __hip_atomic_fetch_add(pcnt + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // Finish tile `tl` (index rot) if this wave owns one of its blocks.
    auto finish_tile = [&](int tl, int rot, const typename S::EpW& e) __attribute__((always_inline)) {
      const int b = my_block(rot);
      if (b < nfin) {   // uniform
        const int q = rot & (NB - 1);
        const bool all_in = lds_wait_eq(pcnt + q, kWaves, p.spin);
        gave_up += all_in ? 0 : 1;
        float* part = red + q * kWaves * MT * 256;
        if (three) {
          finalize_tile3<MT>(p, part, mr, tl, lane, !all_in);
        } else {
          float res[4], add = __builtin_bit_cast(float, 0u);
#pragma unroll
          for (int o = 0; o < 4; ++o) res[o] = elem_to_float(e.v[o], p.x_dtype);
          add = elem_to_float(e.v[4], p.x_dtype);
          if (p.terms == 1) finalize_block<MT, 1>(p, part, mr, b, tl, lane, res, add, !all_in);
          else finalize_block<MT, 2>(p, part, mr, b, tl, lane, res, add, !all_in);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");   // the reads are done
        if (lane == 0) {
          if (__hip_atomic_fetch_add(pfin + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == nfin - 1) {
            __hip_atomic_store(pfin + q, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_store(pcnt + q, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_store(pgen + q, rot + NB, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
      } else {
        asm volatile("" ::"v"(e.v[0]), "v"(e.v[1]), "v"(e.v[2]), "v"(e.v[3]), "v"(e.v[4]));
      }
    };
    auto ep_load = [&](int tl, int rot, typename S::EpW& e) __attribute__((always_inline)) {
      if constexpr (EPI) S::epw_issue(p, tl, three ? MT : my_block(rot), three ? 1 : p.terms, c, li, e);
    };
    // One half: the next tile's codes and scales and this tile's epilogue inputs are issued;
    // this tile is computed from `cur` and `scur` (loaded one half earlier) and its partials
    // are put; then the previous tile is finished, while the next tile's loads are in flight.
    // Putting before finishing keeps a finishing wave from delaying its own partials, which
    // the next tile's finishing wave waits for (a chain that would add one finish per tile).
    // Epilogue inputs are loaded in the half before their use.
    auto half = [&](const typename S::TileRegs& cur, typename S::TileRegs& nxt, const typename S::SbW& scur,
                    typename S::SbW& snxt, const typename S::EpW& eprev, typename S::EpW& ecur, int tl, int next,
                    int rot) __attribute__((always_inline)) {
      S::sbw_issue(p, next, s_lo, c, li, snxt);   // past the last tile: zeros
      S::template load_tile<false, false>(p, next, s_lo, nsw, c, li, nxt);
      ep_load(tl, rot, ecur);
      f4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
      st.compute_regs(s_from, c, scur, cur.dw, acc);
      put(acc, rot);
      if (rot > 0) finish_tile(tl - G, rot - 1, eprev);
      else asm volatile("" ::"v"(eprev.v[0]), "v"(eprev.v[1]), "v"(eprev.v[2]), "v"(eprev.v[3]), "v"(eprev.v[4]));
    };
    // Tiles come in pairs so that the loop is entered again only after the second half: an
    // exit test after the first half that shares a block with the loop test would leave the
    // second set's loads looking unread at the top of the loop.
    const int n = (p.ntiles - tile + G - 1) / G;   // this block's tiles (>= 1: grid <= ntiles)
    typename S::EpW ea, eb;
#pragma unroll
    for (int i = 0; i < 5; ++i) ea.v[i] = eb.v[i] = 0u;
    for (int i = 0; i + 1 < n; i += 2, tile += 2 * G) {
      half(ra, rb, sa, sb, ea, eb, tile, tile + G, i);
      half(rb, ra, sb, sa, eb, ea, tile + G, tile + 2 * G, i + 1);
    }
    if (n & 1) {   // the last tile (index n - 1) is `tile`, in ra / sa
      ep_load(tile, n - 1, eb);
      f4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
      st.compute_regs(s_from, c, sa, ra.dw, acc);
      put(acc, n - 1);
      if (n > 1) finish_tile(tile - G, n - 2, ea);
      finish_tile(tile, n - 1, eb);
    } else {       // the last tile (index n - 1) is tile - G
      finish_tile(tile - G, n - 1, ea);
    }
    if (gave_up != 0 && lane == 0) atomicAdd(p.timeouts, (unsigned int)gave_up);   // all tiles are done
  } else {
    // Long K: rebuild the fragments per chunk.  acc stays in the current chunk's scaled
    // units; switching chunks multiplies by a ratio of powers of two (exact).
    const int nchunks = (p.steps + p.chunk_steps - 1) / p.chunk_steps;
    bool first = true;
    int buf = 0, rot = 0;
    for (int tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x, buf ^= 1, ++rot) {
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
        typename S::StageRegs sr;
        slice(ch, cs0, s_lo, nsw, s_from);
        S::stage_load(p, cs0 * STEPK, min(p.chunk_steps * STEPK, p.K - cs0 * STEPK), tid, sr);
        prepare(ch, first, cs0, s_lo, nsw, s_from, sr, [] {});
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
      // epilogue inputs: slot buf was last read two tiles ago, before the previous barrier
      const long stage_bytes = staging_bytes(p.rows, min(p.chunk_steps * STEPK, p.K));
      uint16_t* epi = reinterpret_cast<uint16_t*>(region + (stage_bytes > merge_bytes(MT) ? stage_bytes : merge_bytes(MT)));
      typename S::EpRegs ep;
      S::ep_issue(p, tile, tid, ep);
      write_partials(acc, buf, red);
      S::ep_commit(p, tid, ep, epi + buf * kEpiSlot);
      finish(tile, rot, buf, epi + buf * kEpiSlot);
    }
  }
}

// Dynamic LDS of a streaming launch: header + max(per-wave staging blocks, merge buffers),
// the layout the kernel carves.
template <int BITS, bool BF16OP, int MT, int NS>
__host__ __device__ constexpr long stream_lds_bytes(int rows, int K) {
  using S = Fused<BITS, BF16OP, MT, NS>;
  const long st = kWaves * S::wave_block_bytes(rows);
  const long mg = (MT <= 2 ? 4L : 2L) * kWaves * MT * 256 * 4;   // the merge buffers
  return kHeaderBytes + (st > mg ? st : mg);
}

// Dynamic LDS of a chunked launch: header + max(staging, merge) + two epilogue-input slots.
__host__ __device__ constexpr long lds_bytes_for(int rows, int kc, int mt) {
  return kHeaderBytes + (staging_bytes(rows, kc) > merge_bytes(mt) ? staging_bytes(rows, kc) : merge_bytes(mt)) +
         2L * kEpiSlot * 2;
}

template <int BITS, bool BF16OP, int MT, bool CHUNKED, int NS, bool EPI, bool NC>
hipError_t launch_nc(const LinParams& p, int grid, size_t lds, hipStream_t s) {
  // Above 64 KiB of dynamic LDS the kernel must opt in once (a host-side attribute).
  static bool opted_in = false;
  if (!opted_in) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&fused_kernel<BITS, BF16OP, MT, CHUNKED, NS, EPI, NC>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e != hipSuccess) return e;
    opted_in = true;
  }
  hipLaunchKernelGGL((fused_kernel<BITS, BF16OP, MT, CHUNKED, NS, EPI, NC>), dim3(grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}
// Normal codes for 4-bit calls without LayerNorm (their rows have no large common part;
// such calls have one operand term per activation row, so MT <= 2); subnormal codes
// otherwise (see convert_codes).
template <int BITS, bool BF16OP, int MT, bool CHUNKED, int NS, bool EPI = false>
hipError_t launch_variant(const LinParams& p, int grid, size_t lds, hipStream_t s) {
  if constexpr (BITS == 4 && MT <= 2) {
    if (!p.ln) return launch_nc<BITS, BF16OP, MT, CHUNKED, NS, EPI, true>(p, grid, lds, s);
  }
  return launch_nc<BITS, BF16OP, MT, CHUNKED, NS, EPI, false>(p, grid, lds, s);
}

// The streaming variant with NS steps per wave, if its staging fits (pieces per lane and
// LDS); hipErrorNotSupported otherwise.
template <int BITS, bool BF16OP, int MT, int NS>
hipError_t try_streaming(const LinParams& p, int grid, hipStream_t s) {
  using S = Fused<BITS, BF16OP, MT, NS>;
  const long pieces = (long)(p.T + (p.ln ? 2 : 0)) * S::W8;
  const long lds = stream_lds_bytes<BITS, BF16OP, MT, NS>(p.rows, p.K);
  if (NS > p.steps || pieces > 64L * S::kWavePieces || lds > kLdsMax) return hipErrorNotSupported;
  if (!p.gateup && (p.res || p.add)) return launch_variant<BITS, BF16OP, MT, false, NS, true>(p, grid, (size_t)lds, s);
  return launch_variant<BITS, BF16OP, MT, false, NS, false>(p, grid, (size_t)lds, s);
}

template <int BITS, bool BF16OP, int MT>
hipError_t launch_one(const LinParams& p, int grid, size_t lds, hipStream_t s) {
  // The streaming variant: every wave a window of NS steps (NS a power of two, at most the
  // fragment budget), the smallest that covers ceil(steps / waves).  It needs rows of whole
  // 64-byte steps and, quantized, K a multiple of 512 and 16-byte aligned scales and biases
  // (each wave's window of a scale row is then one load aligned to its size).
  constexpr int M = max_steps_for(Fmt<BITS>::kMfma, MT);
  const bool whole_steps = ((long)p.K * BITS / 8) % 64 == 0;
  const int G = p.K / 64;
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const bool scales_ok = BITS == 16 || (G % 8 == 0 && a16(p.sc[0]) && a16(p.sc[1]) && a16(p.bi[0]) && a16(p.bi[1]));
  const int need = (p.steps + kWaves - 1) / kWaves;
  if (whole_steps && scales_ok) {
    hipError_t e = hipErrorNotSupported;
    if (need <= 1) e = try_streaming<BITS, BF16OP, MT, 1>(p, grid, s);
    else if (need <= 2) { if constexpr (M >= 2) e = try_streaming<BITS, BF16OP, MT, 2>(p, grid, s); }
    else if (need <= 4) { if constexpr (M >= 4) e = try_streaming<BITS, BF16OP, MT, 4>(p, grid, s); }
    else if (need <= 8) { if constexpr (M >= 8) e = try_streaming<BITS, BF16OP, MT, 8>(p, grid, s); }
    if (e != hipErrorNotSupported) return e;
  }
  return launch_variant<BITS, BF16OP, MT, true, 0>(p, grid, lds, s);
}

}  // namespace qlin
