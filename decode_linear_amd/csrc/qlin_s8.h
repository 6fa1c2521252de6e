// The streaming fused linear on the int8 matrix cores of gfx950 (CDNA4, wave64), for
// 8-bit and 4-bit affine codes.  Shared by the instantiation units qlin_s8_*.hip.
//
// What it computes ([p1] maya-mac src/maya_mac/mlx_kernels.py, `_linear_kernel`):
//   y[t, n] = epi( LN?(x_t) . W_n ),   W[n, k] = q[n, k] * s[n, k/64] + b[n, k/64]
// with LayerNorm folded into the weight stream by the identity of that kernel's docstring,
//   LN(x) . w = rstd * (sum (x - x0) g w - (mean - x0) sum g w) + sum b w,
// the statistics taken in one pass over x shifted by x0 = x[t, 0], and the per-group
// dequantization factored out of the dot product ([p3] mlx-bun 0.0.10 -> 0.0.12,
// fused-decode-kernel.ts, the "qdot pattern"):
//   sum_k (s q_k + b) a_k = s * sum_k q_k a_k + b * sum_k a_k.
//
// How it maps onto CDNA4:
//   * A workgroup of up to 8 waves takes the output tiles blockIdx.x, + grid, ... (16 weight
//     rows each; 8 gate + 8 up rows for gate/up).  Wave w owns a window of GWM quantization
//     groups of K for the whole launch; lane (c, j) reads 16-byte pieces of weight row j
//     (c = lane / 16).  The shape words ride in the pointer arguments that gfx950 preloads
//     into SGPRs, so the first loads go out at wave launch, before any kernel-argument fetch.
//   * Short windows (the activation fragments of the whole window fit in VGPRs): the wave
//     issues every activation piece and then the loads of a ring of R tiles at entry, stages
//     the activations under those loads, and computes the ring slot by slot, issuing the
//     next tile's loads into the slot it has just finished.  Where the tile count is not a
//     multiple of R, the ring starts with all-zero steps: their loads are issued like the
//     others (every path issues the same loads, so a join never waits for loads in flight),
//     and only their arithmetic, which holds no memory operation, is skipped.
//   * Long windows (one tile per workgroup): the window is staged and consumed in chunks of
//     8 groups; the loads of CA chunks are in flight ahead of the chunk being staged.
//   * Exact products on the int8 matrix cores (v_mfma_i32_16x16x64_i8).  Each operand row
//     a (an activation row; with LayerNorm also gamma and beta) becomes, per staging chunk,
//     a 24-bit fixed-point integer X = trunc(a * 2^(16+e)), e the power of two that puts the
//     chunk's max |a| in [64, 128).  X is split into three bytes: the signed top byte and
//     the two low bytes, each taken as (byte - 128).  Codes enter as int8 values: 4-bit codes
//     as they are (0..15), 8-bit codes as q - 128.  One more operand row of ones gives the
//     group's code sum, which restores the byte offsets:
//       sum_k X_k q_k = 65536 C_hi + 256 C_mid + C_lo + 32896 C_ones    (4-bit),
//     with 128 * sum_k X_k added for 8-bit codes.  Every product and every sum inside the
//     MFMA is an exact integer; fp32 rounding enters only per group, where the exact group
//     dot product is converted and scaled by its fp16 scale, and in the sums (a chunk's sum
//     is scaled by 2^-(16+e), exactly, before it joins the lane's partial).
//   * A 16-row MFMA block holds four operand rows: C rows 4r .. 4r + 3 are the three bytes
//     of operand row r and the ones row, so a lane holds all parts of one (row, column)
//     and combines them in registers.
//   * Merge: each wave writes its partial per tile (already in absolute units) to LDS; after
//     the workgroup's single barrier the threads sum the waves' partials in wave order, apply
//     the LayerNorm fold, the epilogue (GELU, residual, constant; or silu(g) * u) and store
//     with one rounding.  No atomics touch data and no wave waits on another before the end,
//     so results are bitwise reproducible and no wait can stall.
#pragma once

#include <type_traits>

#include "qlin_internal.h"

namespace qlin {
namespace s8 {

typedef int i4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef unsigned short us2_t __attribute__((ext_vector_type(2)));

#define QLIN_S8_GLOBAL __attribute__((address_space(1)))
template <typename T> using gp = const T QLIN_S8_GLOBAL*;

// Zero-filled memory that masked lanes load from, so that every path issues the same loads
// (the compiler's wait counts stay exact).  Every masked load ends within its 512 bytes.
static __device__ __attribute__((aligned(256))) uint32_t g_zero[128];

template <typename T> __device__ __forceinline__ gp<T> gaddr(const void* p, long byte_off) {
  return reinterpret_cast<gp<T>>(reinterpret_cast<uintptr_t>(p) + (uintptr_t)byte_off);
}
template <typename T> __device__ __forceinline__ gp<T> zaddr(int byte_off) {
  return reinterpret_cast<gp<T>>(reinterpret_cast<uintptr_t>(g_zero) + (uintptr_t)byte_off);
}

// Arguments needed after the weight loads are issued.  The ones before it in the kernel's
// argument list fit the SGPRs that gfx950 preloads at wave launch (the shape words first),
// so the first loads wait for no kernel-argument fetch.
struct Tail {
  void* y;
  const void* res;   // (T, N) in x's dtype, or null
  const void* add;   // (N,) in x's dtype, or null
  float eps;
  int y_dtype;       // 0 fp32, 1 fp16, 2 bf16
  int act;           // 0 none, 1 GELU
};

// Shape words ride in the top 16 bits of the pointer arguments (device addresses use the
// low 48 bits), so that all of them arrive in the SGPRs preloaded at wave launch:
//   x: K / 64 | (x is bf16) << 15;  w0: T - 1 | gateup << 5;  s0: N & 0xFFFF;
//   b0: N >> 16;  p1: the grid size.
constexpr uint64_t kAddrMask = (uint64_t(1) << kTagShift) - 1;
__host__ __device__ inline uint64_t tag(const void* p, uint32_t v) {
  return (uint64_t)(uintptr_t)p | ((uint64_t)(v & 0xFFFFu) << kTagShift);
}
__device__ __forceinline__ uint32_t tag_of(const void* p) { return (uint32_t)((uint64_t)(uintptr_t)p >> kTagShift); }
template <typename T> __device__ __forceinline__ const T* untag(const void* p) {
  return reinterpret_cast<const T*>((uint64_t)(uintptr_t)p & kAddrMask);
}

// Compile-time shape of one instantiation.
//   MT  16-row MFMA blocks (4 operand rows each: RMAX = 4 MT operand rows)
//   GWM quantization groups in a wave's window (power of two, 2 .. 32)
//   R   ring slots: tiles whose loads are in flight while the wave computes (1 or 2)
//   W   waves per workgroup at most: 8, or 16 for one-tile workgroups (a long K split over
//       more waves, so that more of its loads are in flight at once)
template <int BITS, bool LN, int MT, int GWM, int R, int W>
struct Cfg {
  static constexpr int RMAX = 4 * MT;
  // The operand fragments of the whole window stay in VGPRs when they are few enough;
  // otherwise (a long window, one tile per workgroup) they are staged chunk by chunk,
  // each chunk right before the groups that use it.
  // (16-wave workgroups have half the VGPRs per wave: there only windows of up to 8 groups.)
  static constexpr bool RES = GWM * MT * 4 <= 72 && (W == 8 || GWM <= 8);
  static constexpr int CG = GWM < 8 ? GWM : 8;        // groups staged at once
  static constexpr int NCH = GWM / CG;                 // staging chunks
  static constexpr int AG = RES ? GWM : CG;            // groups of fragments in VGPRs
  // Streamed fragments: chunks whose loads are in flight ahead of the one being staged.  Two
  // measured best on 8-wave workgroups for the MLP's down projection (K = 14336): 17.1 us,
  // against 18.7 with three; windows of 64 groups on four waves were slower still (19.1 us
  // with two, 21.8 with four).  16-wave workgroups take one: with two the registers spill,
  // and the MLP measured 34.2 us against 30.8 with one (32.8 on 8 waves).
  static constexpr int CA = W > 8 ? 1 : 2;
  static constexpr int W8 = 8 * GWM;                   // 8-element pieces per operand row window
  static constexpr int NPX = MT * GWM / 2;             // pieces per lane (RMAX * W8 / 64)
  static constexpr int UPR = GWM >= 8 ? GWM / 8 : 1;   // piece rounds (u) per operand row
  static constexpr int LC = BITS == 8 ? GWM : GWM / 2; // 16-byte code loads per tile and lane
  static constexpr int SBB = 2 * GWM;                  // scale (or bias) bytes per lane and tile
  static constexpr int LS = SBB <= 16 ? 1 : SBB / 16;  // scale/bias loads per tile and lane
  static constexpr int SBW = SBB < 16 ? SBB / 4 : 4;   // dwords per scale/bias load (1, 2 or 4)
  static constexpr int SBD = SBB / 4;                  // scale (bias) dwords per lane
  // LDS: per wave, then the partials of all tiles
  static constexpr int IP = CG * 64 + 16;              // image row pitch (bytes)
  static constexpr int IMG = (3 * RMAX + 1) * IP;      // operand image: 3 byte planes per operand row + a row of ones
  static constexpr int OFF_MAX = 0;                    // rowmax[RMAX] (u32)
  static constexpr int OFF_ST = OFF_MAX + RMAX * 4;    // LN: S1, S2 [RMAX][GWM][2]
  static constexpr int OFF_IMG = (OFF_ST + (LN ? RMAX * GWM * 8 : 0) + 15) / 16 * 16;
  static constexpr int WAVE_BYTES = OFF_IMG + IMG;
  static constexpr int PMAX = W > 8 ? 1 : max_tiles(BITS, LN, MT, GWM);   // tiles of one workgroup, at most
  static constexpr int PART_BYTES = PMAX * W * MT * 256;
  static constexpr int LDS_BYTES = W * WAVE_BYTES + PART_BYTES;
  static_assert(GWM >= 2 && (GWM & (GWM - 1)) == 0 && GWM <= 32, "windows of 2..32 groups");
  static_assert(PMAX >= 1, "an instantiated shape");
  static_assert(W == 8 || (W == 16 && R == 1), "8 waves, or 16 for one tile");
  static_assert(RES || (R == 1 && PMAX == 1), "streamed fragments serve one tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// 8 consecutive 16-bit elements of a 16-byte piece, widened to fp32.
__device__ __forceinline__ void widen8(const u4_t r, bool bf, float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf ? bf16_lo(r[i]) : f16_lo(r[i]);
    v[2 * i + 1] = bf ? bf16_hi(r[i]) : f16_hi(r[i]);
  }
}

template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Reductions over aligned groups of 8 lanes (xor 1, xor 2, then the mirrored half-row):
// every lane of a group ends with the group's value, and the order is fixed.
__device__ __forceinline__ float sum8f(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v;
}
__device__ __forceinline__ int sum8i(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x141>(v);
  return v;
}
__device__ __forceinline__ uint32_t max8u(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<0xB1>((int)v));
  v = max(v, (uint32_t)dpp_i<0x4E>((int)v));
  v = max(v, (uint32_t)dpp_i<0x141>((int)v));
  return v;
}

// Max over aligned groups of N lanes (N a power of two, 8..64): DPP moves within 16-lane
// rows (xor 1, xor 2, the mirrored half-row, the mirrored row), then the gfx950 row swaps
// (v_permlane16_swap pairs rows 0-1 and 2-3, v_permlane32_swap the two halves).
// Level L of group_max alone (levels 0-2: max8u's moves; 3: the mirrored row; 4, 5: the row
// swaps), so that several values can be reduced level by level with independent moves.
template <int N, int L> __device__ __forceinline__ uint32_t group_max_level(uint32_t v) {
  if constexpr (L == 0) return max(v, (uint32_t)dpp_i<0xB1>((int)v));
  else if constexpr (L == 1) return max(v, (uint32_t)dpp_i<0x4E>((int)v));
  else if constexpr (L == 2) return max(v, (uint32_t)dpp_i<0x141>((int)v));
  else if constexpr (L == 3) return N >= 16 ? max(v, (uint32_t)dpp_i<0x140>((int)v)) : v;
  else if constexpr (L == 4) {
    if constexpr (N < 32) return v;
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max((uint32_t)r[0], (uint32_t)r[1]);
  } else {
    if constexpr (N < 64) return v;
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((uint32_t)r[0], (uint32_t)r[1]);
  }
}
template <int N> __device__ __forceinline__ uint32_t group_max(uint32_t v) {
  static_assert(N >= 8 && N <= 64, "groups of 8..64 lanes");
  v = max8u(v);
  if constexpr (N >= 16) v = max(v, (uint32_t)dpp_i<0x140>((int)v));
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

// Window exponent e of an operand row from its max |a| (bit pattern): max * 2^e in
// [64, 128).  A zero row takes 0; the exponent is clamped so that 2^-(16+e) stays normal.
__device__ __forceinline__ int row_exp(uint32_t amax_bits) {
  const int be = (int)(amax_bits >> 23);
  if (amax_bits == 0u) return 0;
  const int e = 6 - (be - 127);
  return e > 100 ? 100 : e;
}

// Bytes of four 24-bit integers X0..X3 (two's complement in int32): term 0 = the signed
// top bytes, terms 1 and 2 = bytes 1 and 0 minus 128 (as int8: the byte xor 0x80).
__device__ __forceinline__ void split4(int x0, int x1, int x2, int x3, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t p01 = __builtin_amdgcn_perm((uint32_t)x1, (uint32_t)x0, 0x05010400u);   // x0.b0 x1.b0 x0.b1 x1.b1
  const uint32_t p23 = __builtin_amdgcn_perm((uint32_t)x3, (uint32_t)x2, 0x05010400u);
  const uint32_t q01 = __builtin_amdgcn_perm((uint32_t)x1, (uint32_t)x0, 0x07030602u);   // x0.b2 x1.b2 x0.b3 x1.b3
  const uint32_t q23 = __builtin_amdgcn_perm((uint32_t)x3, (uint32_t)x2, 0x07030602u);
  lo = __builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x80808080u;    // p01.b0 p01.b1 p23.b0 p23.b1
  mid = __builtin_amdgcn_perm(p23, p01, 0x07060302u) ^ 0x80808080u;   // p01.b2 p01.b3 p23.b2 p23.b3
  hi = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
}

__device__ __forceinline__ void store_y(void* y, int dtype, long idx, float v) {
  if (dtype == 0) reinterpret_cast<float*>(y)[idx] = v;
  else if (dtype == 1) reinterpret_cast<_Float16*>(y)[idx] = (_Float16)v;
  else reinterpret_cast<__bf16*>(y)[idx] = (__bf16)v;
}
__device__ __forceinline__ float elem(uint32_t h, bool bf) {
  return bf ? __builtin_bit_cast(float, h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int BITS, bool LN, int MT, int GWM, int R, int W>
struct Kern {
  using C = Cfg<BITS, LN, MT, GWM, R, W>;

  // One tile's loads: the codes of this wave's window and the scales (even lane groups) or
  // biases (odd lane groups) of its groups.
  struct TileRegs {
    u4_t code[C::LC];
    uint32_t sb[C::LS * C::SBW];
  };

  // Issue the loads of chunk ch (groups [ch CG, (ch + 1) CG) of the window) of tile `tile`:
  // the chunk's scales (even lane groups) or biases (odd lane groups), then its codes.  Rows
  // past N and tiles past the last read zeros.
  __device__ __forceinline__ static void issue_chunk(TileRegs& r, int ch, int tile, int ntiles, const uint8_t* w0,
                                                     const void* w1, const uint16_t* s0, const void* s1,
                                                     const uint16_t* b0, const void* b1, int N, int gateup,
                                                     int row_bytes, int G, int g_lo, int c, int j) {
    int proj, n;
    if (gateup) { proj = j >> 3; n = tile * 8 + (j & 7); }
    else { proj = 0; n = tile * 16 + j; }
    const bool valid = tile < ntiles && n < N;
    const void* sp = (c & 1) ? (proj ? b1 : (const void*)b0) : (proj ? s1 : (const void*)s0);
    const long sbo = ((long)n * G + g_lo) * 2;
    if constexpr (C::SBW == 4) {   // one 16-byte load per chunk of 8 groups
      const bool ok = valid && g_lo + ch * 8 < G;
      const u4_t v = *(ok ? gaddr<u4_t>(sp, sbo + 16L * ch) : zaddr<u4_t>(0));
#pragma unroll
      for (int i = 0; i < 4; ++i) r.sb[4 * ch + i] = v[i];
    } else if constexpr (C::SBW == 2) {
      const u2_t v = *(valid ? gaddr<u2_t>(sp, sbo) : zaddr<u2_t>(0));
      r.sb[0] = v[0];
      r.sb[1] = v[1];
    } else {
      r.sb[0] = *(valid ? gaddr<uint32_t>(sp, sbo) : zaddr<uint32_t>(0));
    }
    const void* wb = proj ? w1 : (const void*)w0;
    const long rowoff = (long)n * row_bytes;
    constexpr int LCC = C::LC / C::NCH;   // code loads per chunk
#pragma unroll
    for (int qq = 0; qq < LCC; ++qq) {
      const int q = ch * LCC + qq;
      // 8-bit: group g_lo + q, bytes 16c of it; 4-bit: step g_lo/2 + q (groups 2 step + c/2)
      const int g = BITS == 8 ? g_lo + q : g_lo + 2 * q + (c >> 1);
      const long off = BITS == 8 ? rowoff + 64L * (g_lo + q) + 16 * c : rowoff + 32L * (g_lo + 2 * q) + 16 * c;
      const bool ok = valid && g < G;
      r.code[q] = *(ok ? gaddr<u4_t>(wb, off) : zaddr<u4_t>(16 * c));
    }
  }

  // B operand of group gg of the window (16 int8 codes of column j, this lane's k-quarter).
  // 4-bit: after the lane-half exchange (see compute), dwords 0-1 hold the even group and
  // dwords 2-3 the odd group of a step; nibbles split into low (even k) and high (odd k).
  __device__ __forceinline__ static i4_t operand_b(const u4_t d, int gg) {
    if constexpr (BITS == 8) {
      return (i4_t){(int)(d[0] ^ 0x80808080u), (int)(d[1] ^ 0x80808080u), (int)(d[2] ^ 0x80808080u),
                    (int)(d[3] ^ 0x80808080u)};
    } else {
      const uint32_t a = (gg & 1) ? d[2] : d[0], b = (gg & 1) ? d[3] : d[1];
      return (i4_t){(int)(a & 0x0F0F0F0Fu), (int)((a >> 4) & 0x0F0F0F0Fu), (int)(b & 0x0F0F0F0Fu),
                    (int)((b >> 4) & 0x0F0F0F0Fu)};
    }
  }
};

// Inverse of the 4-bit k order: the lane group that feeds 16-code run (k >> 4) of a group.
// (0, 1, 2, 3 -> 0, 2, 1, 3: the two bits swapped, in arithmetic so that no branch is made of it)
__device__ __forceinline__ constexpr int kq4(int run) { return ((run & 1) << 1) | ((run >> 1) & 1); }

template <int BITS, bool LN, int MT, int GWM, int R, int W, bool XBF>
__global__ __attribute__((amdgpu_flat_work_group_size(1, W * 64))) void s8_kernel(
    const void* xt, const void* w0t, const void* s0t, const void* b0t, const void* p1t, const void* p2t,
    const void* p3t, const Tail tail) {
  using C = Cfg<BITS, LN, MT, GWM, R, W>;
  using Kx = Kern<BITS, LN, MT, GWM, R, W>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS_BYTES];

  const uint32_t tx = tag_of(xt), tw = tag_of(w0t);
  const int G = (int)(tx & 0x7FFFu), K = G << 6;
  constexpr bool xbf = XBF;   // the activations' dtype (bf16, else fp16) is part of the instantiation
  const int T = (int)(tw & 31u) + 1;
  const int gateup = (int)((tw >> 5) & 1u);
  const int N = (int)(tag_of(s0t) | (tag_of(b0t) << 16));
  const int grid = (int)tag_of(p1t);
  const uint16_t* x = untag<uint16_t>(xt);
  const uint8_t* w0 = untag<uint8_t>(w0t);
  const uint16_t* s0 = untag<uint16_t>(s0t);
  const uint16_t* b0 = untag<uint16_t>(b0t);
  const void* p1 = untag<void>(p1t);
  const void* p2 = untag<void>(p2t);
  const void* p3 = untag<void>(p3t);
  const int row_bytes = K * BITS / 8;
  const int ntiles = gateup ? (N + 7) >> 3 : (N + 15) >> 4;
  const int tid = threadIdx.x, lane = tid & 63, c = lane >> 4, j = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int waves = (G + GWM - 1) / GWM;
  const int g_lo = wv * GWM;
  const int ntw = (ntiles - (int)blockIdx.x + grid - 1) / grid;   // tiles of this workgroup (1 .. PMAX)
  const int RS = T + (LN ? 2 : 0);                                   // operand rows in use
  const uint16_t* gam = LN ? static_cast<const uint16_t*>(p1) : nullptr;
  const uint16_t* bet = LN ? static_cast<const uint16_t*>(p2) : nullptr;

  unsigned char* wbase = lds + wv * C::WAVE_BYTES;
  uint32_t* rowmax = reinterpret_cast<uint32_t*>(wbase + C::OFF_MAX);
  float* sts = reinterpret_cast<float*>(wbase + C::OFF_ST);
  unsigned char* img = wbase + C::OFF_IMG;
  float* parts = reinterpret_cast<float*>(lds + W * C::WAVE_BYTES);

  // ---- 1. loads -------------------------------------------------------------------
  // Operand pieces: piece p = lane + 64 u is operand row rho = p / W8, piece kp = p % W8 of
  // the window (elements 64 g_lo + 8 kp .. + 7), in staging chunk (u mod UPR) when the window
  // has several chunks.  Pieces past the rows in use or past K read zeros.
  u4_t raw[C::NPX];
  // LayerNorm: gamma at each piece's k, and x[rho, 0] (the shift of each piece's row).  When
  // a row's pieces divide the wave (W8 | 64), every piece of a lane covers the same k: gamma
  // is loaded and widened once per lane.
  constexpr bool GSH = LN && (64 % C::W8 == 0);
  u4_t graw[LN ? (GSH ? 1 : C::NPX) : 1];
  uint32_t x0r[LN ? C::NPX : 1];
  auto load_pieces = [&](int ch) __attribute__((always_inline)) {
    if constexpr (GSH) {
      const int kp = lane % C::W8;
      graw[0] = *(g_lo + (kp >> 3) < G ? gaddr<u4_t>(gam, (64L * g_lo + 8 * kp) * 2) : zaddr<u4_t>(0));
    }
#pragma unroll
    for (int u = 0; u < C::NPX; ++u) {
      if (C::NCH > 1 && (u % C::UPR) != ch) continue;
      const int p = lane + 64 * u, rho = p / C::W8, kp = p % C::W8;
      const int g = g_lo + (kp >> 3);
      const bool real = rho < RS && g < G;
      const long k = 64L * g_lo + 8 * kp;
      const void* src = x;
      long off = ((long)rho * K + k) * 2;
      if constexpr (LN) {
        if (rho >= T) { src = rho == T ? (const void*)gam : (const void*)bet; off = k * 2; }
      }
      raw[u] = *(real ? gaddr<u4_t>(src, off) : zaddr<u4_t>(0));
      if constexpr (LN) {
        if constexpr (!GSH) graw[u] = *(real ? gaddr<u4_t>(gam, k * 2) : zaddr<u4_t>(0));
        x0r[u] = *(rho < T ? gaddr<uint16_t>(x, (long)rho * K * 2) : zaddr<uint16_t>(0));
      }
    }
  };

  // Tiles: a ring of R slots.  Step q of the workgroup's sequence carries its tile q - z; the
  // z = (R - ntw mod R) mod R leading steps carry zeros: their loads (of zeros) are issued
  // like every other step's, so the loads in flight are the same on every path, and only
  // their arithmetic is skipped (a branch around memory operations would make the compiler
  // wait for every load in flight where the paths join).  Skipping it lets the first real
  // tile start as soon as the staging is done: C4 16.4-16.5 -> 16.2-16.4 us.
  typename Kx::TileRegs tr[R];
  const int nq = (ntw + R - 1) / R * R;   // steps
  const int z = nq - ntw;
  auto tile_of = [&](int q) __attribute__((always_inline)) {
    return (q < z || q >= nq) ? ntiles : (int)blockIdx.x + (q - z) * grid;
  };
  // Workgroups of several tiles with windows inside K (at most 8 groups, and the host admits
  // them only when they divide G): the lane's code and scale/bias rows are addressed from
  // bases fixed for the launch, a tile's row by one multiply-add (clamped to the last row
  // of the matrix: a partial last tile's extra rows are loaded but never stored), and every
  // load of the tile by an immediate offset from it.  Steps without a tile read the zero
  // line.  (C2 8.10-8.17 -> 7.73-7.87 us, the MLP 25.8 -> 25.5; one-tile launches address
  // their tile once and gained nothing from it: C3 10.1 -> 10.2, the shard shape 5.7 -> 5.6.)
  constexpr bool LANE_BASES = GWM <= 8 && R >= 2;
  const int jrow = gateup ? (j & 7) : j;
  const bool second = gateup && (j >> 3);   // the up projection's rows
  const uint8_t* cbase = (second ? static_cast<const uint8_t*>(p1) : w0) + (BITS == 8 ? 64 : 32) * g_lo + 16 * c;
  const uint16_t* sbase =
      ((c & 1) ? (second ? static_cast<const uint16_t*>(p3) : b0) : (second ? static_cast<const uint16_t*>(p2) : s0)) +
      g_lo;
  auto issue_tile = [&](typename Kx::TileRegs& r, int tile) __attribute__((always_inline)) {
    if constexpr (LANE_BASES) {
      const bool ok = tile < ntiles;   // uniform
      const int n = min(tile * (gateup ? 8 : 16) + jrow, N - 1);
      const gp<u4_t> ca = ok ? gaddr<u4_t>(cbase, (uint64_t)(uint32_t)n * (uint32_t)row_bytes) : zaddr<u4_t>(16 * c);
      const gp<uint32_t> sa = ok ? gaddr<uint32_t>(sbase, (uint64_t)(uint32_t)n * (uint32_t)(2 * G)) : zaddr<uint32_t>(0);
      if constexpr (C::SBW == 4) {
#pragma unroll
        for (int ch = 0; ch < C::NCH; ++ch) {
          const u4_t v = *reinterpret_cast<gp<u4_t>>(sa + 4 * ch);
#pragma unroll
          for (int i = 0; i < 4; ++i) r.sb[4 * ch + i] = v[i];
        }
      } else if constexpr (C::SBW == 2) {
        const u2_t v = *reinterpret_cast<gp<u2_t>>(sa);
        r.sb[0] = v[0];
        r.sb[1] = v[1];
      } else {
        r.sb[0] = *sa;
      }
#pragma unroll
      for (int q = 0; q < C::LC; ++q) r.code[q] = ca[4 * q];
    } else {
#pragma unroll
      for (int ch = 0; ch < C::NCH; ++ch)
        Kx::issue_chunk(r, ch, tile, ntiles, w0, p1, s0, p2, b0, p3, N, gateup, row_bytes, G, g_lo, c, j);
    }
  };
  if constexpr (C::RES) {
    // every operand piece, then the ring's first tiles (staging waits for its pieces only:
    // loads complete in order)
#pragma unroll
    for (int ch = 0; ch < C::NCH; ++ch) load_pieces(ch);
#pragma unroll
    for (int r = 0; r < R; ++r) issue_tile(tr[r], tile_of(r));
  } else {
    // one tile, chunk by chunk: each chunk's operand pieces, then its scales, biases and codes;
    // CA chunks ahead (the rest are issued as chunks complete: a wave whose loads fill the
    // memory queue stalls at the issue and could not stage what has arrived)
#pragma unroll
    for (int ch = 0; ch < (C::NCH < C::CA ? C::NCH : C::CA); ++ch) {
      load_pieces(ch);
      Kx::issue_chunk(tr[0], ch, tile_of(0), ntiles, w0, p1, s0, p2, b0, p3, N, gateup, row_bytes, G, g_lo, c, j);
    }
  }

  // epilogue inputs of this thread's first output (loaded now, used at the end)
  const int nthreads = waves * 64;
  const int per_tile = gateup ? 8 * T : 16 * T;
  uint32_t res0 = 0u, add0 = 0u;
  {
    const int o = tid, i = o / per_tile, rem = o - i * per_tile;
    const int t = gateup ? rem >> 3 : rem >> 4, jj = gateup ? rem & 7 : rem & 15;
    const int tile = (int)blockIdx.x + i * grid;
    const int n = gateup ? tile * 8 + jj : tile * 16 + jj;
    const bool ok = i < ntw && n < N && !gateup;
    res0 = *((ok && tail.res) ? gaddr<uint16_t>(tail.res, ((long)t * N + n) * 2) : zaddr<uint16_t>(0));
    add0 = *((ok && tail.add) ? gaddr<uint16_t>(tail.add, (long)n * 2) : zaddr<uint16_t>(0));
  }

  // ---- 2. staging, per chunk ----------------------------------------------------------
  // Each (operand row, chunk) takes its own exponent e: the chunk's max |a| * 2^e lies in
  // [64, 128).  Within a chunk the lane sums the groups' scaled exact integer dot products
  // in units of 2^-(16 + e) of its operand row; the chunk's sum is then multiplied by
  // 2^-(16 + e) (an exact power of two) into the lane's partial in absolute units.
  float gms[GSH ? 8 : 1];   // the lane's gamma values (shared by its pieces), widened at the first staging
  auto values = [&](int u, float a[8], float dsh[8]) __attribute__((always_inline)) {
    const int p = lane + 64 * u, rho = p / C::W8;
    widen8(raw[u], xbf, a);
    if constexpr (LN) {
      float gm[8];
      if constexpr (GSH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) gm[e] = gms[e];
      } else {
        widen8(graw[u], xbf, gm);
      }
      const float x0 = elem(x0r[u] & 0xFFFFu, xbf);
      const bool xr = rho < T;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dsh[e] = a[e] - x0;
        a[e] = xr ? dsh[e] * gm[e] : a[e];
      }
    }
  };
  float unit[C::NCH][MT];   // 2^-(16 + e) of this lane's C-row operand row (4 mt + c), per chunk
  bool poison[MT];          // a non-finite operand value: the row's outputs become NaN
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) poison[mt] = false;
  // the ones row (operand rows 4r + 3 of every block read it)
  if (lane < C::CG * 8) *reinterpret_cast<u2_t*>(img + 3 * C::RMAX * C::IP + 8 * lane) = (u2_t){0x01010101u, 0x01010101u};
  i4_t af[C::AG][MT];
  float gxf[C::AG][MT];
  const int arow = lane & 15, akq = lane >> 4;   // A operand: row arow, k-quarter akq
  // Pass 1: the max |a| of each (row, chunk) over a group of min(W8, 64) lanes (a chunk of a
  // longer row fills one round u), published by one lane; with LN also the shifted sums.
  // Pass 2: X = trunc(a 2^(16 + e)) split into its three bytes, written in the order lane
  // group kq reads them (image row 3 rho + v: v = 0 top bytes, 1 middle, 2 low; 8-bit
  // k = 16 kq + b, 4-bit k = {0, 32, 16, 48}[kq] + 8 (b >> 3) + 2 (b & 3) + ((b >> 2) & 1)).
  // Then the chunk's fragments into slots [base, base + CG), and their group sums of X.
  // With LayerNorm and several MFMA blocks, pass 1 keeps its values for pass 2 (registers
  // are free there, and recomputing the shifted, gamma-scaled values is most of the staging).
  constexpr bool KEEP = LN && MT >= 2;
  float kept[KEEP ? C::NPX : 1][8];
  auto stage = [&](int ch, int base) __attribute__((always_inline)) {
    if constexpr (GSH) widen8(graw[0], xbf, gms);
    uint32_t rmx[C::NPX];
#pragma unroll
    for (int u = 0; u < C::NPX; ++u) {
      if (C::NCH > 1 && (u % C::UPR) != ch) continue;
      const int p = lane + 64 * u, rho = p / C::W8, kp = p % C::W8;
      uint32_t m;
      if constexpr (LN) {
        float a[8], dsh[8];
        values(u, a, dsh);
        if constexpr (KEEP) {
#pragma unroll
          for (int e = 0; e < 8; ++e) kept[u][e] = a[e];
        }
        m = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, __builtin_bit_cast(uint32_t, a[e]) & 0x7FFFFFFFu);
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { s1 += dsh[e]; s2 += dsh[e] * dsh[e]; }
        s1 = sum8f(s1);
        s2 = sum8f(s2);
        const int g = g_lo + (kp >> 3);
        if ((lane & 7) == 0 && rho < T) {
          const bool real = g < G;
          sts[(rho * GWM + (kp >> 3)) * 2] = real ? s1 : 0.0f;
          sts[(rho * GWM + (kp >> 3)) * 2 + 1] = real ? s2 : 0.0f;
        }
      } else {
        // magnitudes of the 16-bit values, two per dword (their bit patterns order like the
        // values), widened once at the end
        us2_t hm = __builtin_bit_cast(us2_t, raw[u][0] & 0x7FFF7FFFu);
#pragma unroll
        for (int i = 1; i < 4; ++i) hm = __builtin_elementwise_max(hm, __builtin_bit_cast(us2_t, raw[u][i] & 0x7FFF7FFFu));
        const uint32_t h = max((uint32_t)hm[0], (uint32_t)hm[1]);
        m = xbf ? h << 16 : __builtin_bit_cast(uint32_t, f16_lo(h));
      }
      if constexpr (W == 8) {
        rmx[u] = m;
      } else {
        rmx[u] = group_max<(C::W8 < 64 ? C::W8 : 64)>(m);
        rowmax[rho] = rmx[u];
      }
    }
    // the max over each group of min(W8, 64) lanes, level by level over the chunk's pieces (the
    // moves of one level are independent; 16-wave workgroups, at 128 VGPRs, reduce each piece
    // as it is formed instead); every lane of a group then holds the group's max, so all of
    // them store it
    constexpr int GM = C::W8 < 64 ? C::W8 : 64;
    auto level = [&](auto L) __attribute__((always_inline)) {
      if constexpr (W != 8) return;
#pragma unroll
      for (int u = 0; u < C::NPX; ++u) {
        if (C::NCH > 1 && (u % C::UPR) != ch) continue;
        rmx[u] = group_max_level<GM, decltype(L)::value>(rmx[u]);
      }
    };
    level(std::integral_constant<int, 0>{});
    level(std::integral_constant<int, 1>{});
    level(std::integral_constant<int, 2>{});
    level(std::integral_constant<int, 3>{});
    level(std::integral_constant<int, 4>{});
    level(std::integral_constant<int, 5>{});
    if constexpr (W == 8) {
#pragma unroll
      for (int u = 0; u < C::NPX; ++u) {
        if (C::NCH > 1 && (u % C::UPR) != ch) continue;
        rowmax[(lane + 64 * u) / C::W8] = rmx[u];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t mb = rowmax[4 * mt + c];
      unit[ch][mt] = __builtin_bit_cast(float, (uint32_t)(127 - 16 - row_exp(mb)) << 23);
      poison[mt] = poison[mt] || (mb >> 23) >= 255u;
    }
#pragma unroll
    for (int u = 0; u < C::NPX; ++u) {
      if (C::NCH > 1 && (u % C::UPR) != ch) continue;
      const int p = lane + 64 * u, rho = p / C::W8, kp = p % C::W8;
      const int gg = kp >> 3, pp = kp & 7;
      float a[8], dsh[8];
      if constexpr (KEEP) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = kept[u][e];
      } else {
        values(u, a, dsh);
      }
      // a row max reduced over the whole wave is uniform: its exponent is scalar work
      const uint32_t rm = (C::W8 >= 64) ? (uint32_t)__builtin_amdgcn_readfirstlane((int)rmx[u]) : rmx[u];
      const int ex = 16 + row_exp(rm);
      int X[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) X[e] = (int)__builtin_amdgcn_ldexpf(a[e], ex);
      uint32_t h0, m0, l0, h1, m1, l1;
      if constexpr (BITS == 8) {
        split4(X[0], X[1], X[2], X[3], h0, m0, l0);
        split4(X[4], X[5], X[6], X[7], h1, m1, l1);
      } else {
        split4(X[0], X[2], X[4], X[6], h0, m0, l0);
        split4(X[1], X[3], X[5], X[7], h1, m1, l1);
      }
      const int kq = BITS == 8 ? (pp >> 1) : kq4(pp >> 1);
      const int col = (gg % C::CG) * 64 + kq * 16 + 8 * (pp & 1);
      *reinterpret_cast<u2_t*>(img + (3 * rho + 0) * C::IP + col) = (u2_t){h0, h1};
      *reinterpret_cast<u2_t*>(img + (3 * rho + 1) * C::IP + col) = (u2_t){m0, m1};
      *reinterpret_cast<u2_t*>(img + (3 * rho + 2) * C::IP + col) = (u2_t){l0, l1};
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < C::CG; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int rho = 4 * mt + (arow >> 2), v = arow & 3;
        af[base + q][mt] = *reinterpret_cast<const i4_t*>(img + (v < 3 ? 3 * rho + v : 3 * C::RMAX) * C::IP + q * 64 +
                                                            akq * 16);
      }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    // Group sums of X: the fragments against a B of ones give, in this lane's C rows, the
    // byte sums of its operand row (and 64 for the ones row); X = 65536 hi + 256 mid + lo +
    // 32896 per element.
    const i4_t ones = (i4_t){0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
    for (int q = 0; q < C::CG; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i4_t cs = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[base + q][mt], ones, (i4_t){0, 0, 0, 0}, 0, 0, 0);
        gxf[base + q][mt] = fmaf((float)cs[0], 65536.0f, fmaf((float)cs[1], 256.0f, (float)cs[2] + 2105344.0f));
      }
  };

  // ---- 3. the tiles --------------------------------------------------------------
  // acc (per block): this lane's partial of (operand row 4 mt + c, column j), absolute units.
  // accc: the chunk's sums in units of 2^-(16 + e) (the chunk's exponent); chunk_step scales
  // them to absolute units once (an exact power of two).  A group's products come from
  // group_mfma; group_sum folds them in (split so that a pair of groups issues its MFMAs
  // before either result is read, which hides the MFMA latency).
  auto group_mfma = [&](const u4_t& d, int gg, int slot, i4_t cc[MT]) __attribute__((always_inline)) {
    const i4_t bop = Kx::operand_b(d, gg);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      cc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[slot][mt], bop, (i4_t){0, 0, 0, 0}, 0, 0, 0);
  };
  auto group_sum = [&](const typename Kx::TileRegs& r, int gg, int slot, const i4_t cc[MT],
                       float accc[MT]) __attribute__((always_inline)) {
    // scale and bias of group gg for column j: dword gg/2 of the lane's scales (biases), half gg&1
    const uint32_t sw = r.sb[gg >> 1];
    const auto sbp = __builtin_amdgcn_permlane16_swap(sw, sw, false, false);
    const uint32_t swd = (uint32_t)sbp[0], bwd = (uint32_t)sbp[1];
    const float s = (gg & 1) ? f16_hi(swd) : f16_lo(swd);
    const float b = (gg & 1) ? f16_hi(bwd) : f16_lo(bwd);
    const float bb = BITS == 8 ? fmaf(128.0f, s, b) : b;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // sum X q = 65536 C_hi + 256 C_mid + C_lo + 32896 C_ones: two exact integer parts
      // (|C| < 2^21 for every part, |C_ones| <= 8192), one rounding each, one fma
      const int t1 = cc[mt][0] * 256 + cc[mt][1];
      const int t2 = cc[mt][2] + __mul24(cc[mt][3], 32896);
      const float cf = fmaf((float)t1, 256.0f, (float)t2);
      accc[mt] = fmaf(s, cf, accc[mt]);
      accc[mt] = fmaf(bb, gxf[slot][mt], accc[mt]);
    }
  };
  // the code dword set of group gg (4-bit: exchange lane halves once per step)
  auto codes_of = [&](const typename Kx::TileRegs& r, int gg) __attribute__((always_inline)) {
    if constexpr (BITS == 8) {
      return r.code[gg];
    } else {
      const u4_t d = r.code[gg >> 1];
      const auto e02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
      const auto e13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
      return (u4_t){(uint32_t)e02[0], (uint32_t)e13[0], (uint32_t)e02[1], (uint32_t)e13[1]};
    }
  };
  // the groups of chunk ch of one tile, fragments from slots [base, base + CG)
  auto chunk_step = [&](const typename Kx::TileRegs& r, int ch, int base, float acc[MT]) __attribute__((always_inline)) {
    float accc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) accc[mt] = 0.0f;
#pragma unroll
    for (int q = 0; q < C::CG; q += 2) {   // CG is even (2 .. 8)
      const int gg = ch * C::CG + q;
      i4_t c0[MT], c1[MT];
      if constexpr (BITS == 4) {   // one step holds both groups
        const u4_t dd = codes_of(r, gg);
        group_mfma(dd, gg, base + q, c0);
        group_mfma(dd, gg + 1, base + q + 1, c1);
      } else {
        group_mfma(codes_of(r, gg), gg, base + q, c0);
        group_mfma(codes_of(r, gg + 1), gg + 1, base + q + 1, c1);
      }
      group_sum(r, gg, base + q, c0, accc);
      group_sum(r, gg + 1, base + q + 1, c1, accc);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = fmaf(unit[ch][mt], accc[mt], acc[mt]);
  };
  auto put_partial = [&](int i, const float acc[MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      parts[((i * W + wv) * MT + mt) * 64 + lane] = poison[mt] ? __builtin_nanf("") : acc[mt];
  };

  if constexpr (C::RES) {
#pragma unroll
    for (int ch = 0; ch < C::NCH; ++ch) stage(ch, ch * C::CG);
    for (int q0 = 0; q0 < nq; q0 += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int q = q0 + r;
        if (q >= z) {   // a leading zero step is not computed (no memory operation in the branch)
          float acc[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] = 0.0f;
#pragma unroll
          for (int ch = 0; ch < C::NCH; ++ch) chunk_step(tr[r], ch, ch * C::CG, acc);
          put_partial(q - z, acc);
        }
        issue_tile(tr[r], tile_of(q + R));
        // Two waves share each SIMD and the older one wins issue: left alone it runs ahead,
        // its loads go out earlier, and at the end it waits for the younger at the merge
        // (about 2 us on the SwiGLU shape).  A workgroup barrier per step (no memory wait;
        // every wave runs the same steps) keeps the waves in step where there are many steps.
        if constexpr (W == 8) {
          if (nq >= 4) __builtin_amdgcn_s_barrier();
        }
      }
    }
  } else {
    float acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = 0.0f;
#pragma unroll
    for (int ch = 0; ch < C::NCH; ++ch) {
      stage(ch, 0);
      chunk_step(tr[0], ch, 0, acc);
      if (ch + C::CA < C::NCH) {
        load_pieces(ch + C::CA);
        Kx::issue_chunk(tr[0], ch + C::CA, tile_of(0), ntiles, w0, p1, s0, p2, b0, p3, N, gateup, row_bytes, G, g_lo,
                        c, j);
      }
    }
    put_partial(0, acc);   // one tile: ntw == 1
  }

  // ---- 6. merge, LayerNorm fold, epilogue, store -------------------------------------
  __syncthreads();
  const float inv_k = 1.0f / (float)K;
  for (int o = tid; o < ntw * per_tile; o += nthreads) {
    const int i = o / per_tile, rem = o - i * per_tile;
    const int t = gateup ? rem >> 3 : rem >> 4, jj = gateup ? rem & 7 : rem & 15;
    const int tile = (int)blockIdx.x + i * grid;
    const int n = gateup ? tile * 8 + jj : tile * 16 + jj;
    if (n >= N) continue;
    // the waves' partials in wave order; the loops run over the instantiation's W waves (the
    // reads are all in the partials' LDS), and a wave past the launch's adds zero
    auto read_parts = [&](int rho, int col, float pw[W]) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < W; ++w) pw[w] = parts[((i * W + w) * MT + (rho >> 2)) * 64 + (rho & 3) * 16 + col];
    };
    auto sum_parts = [&](const float pw[W]) __attribute__((always_inline)) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) v += w < waves ? pw[w] : 0.0f;
      return v;
    };
    auto merged = [&](int rho, int col) __attribute__((always_inline)) {
      float pw[W];
      read_parts(rho, col, pw);
      return sum_parts(pw);
    };
    // the gate and up rows' partials are read together, on every path (the empty asm takes
    // the up values, so that the compiler cannot sink their reads into the gate/up branch)
    float pv[W], pu[W];
    read_parts(t, jj, pv);
    read_parts(t, gateup ? jj + 8 : jj, pu);
#pragma unroll
    for (int w = 0; w < W; ++w) asm volatile("" ::"v"(pu[w]));
    float v = sum_parts(pv);
    float u = gateup ? sum_parts(pu) : 0.0f;
    if constexpr (LN) {
      float s1 = 0.0f, s2 = 0.0f;
      for (int w = 0; w < waves; ++w) {
        const float* st = reinterpret_cast<const float*>(lds + w * C::WAVE_BYTES + C::OFF_ST);
        for (int q = 0; q < GWM; ++q) { s1 += st[(t * GWM + q) * 2]; s2 += st[(t * GWM + q) * 2 + 1]; }
      }
      const float m = s1 * inv_k;
      const float var = fmaxf(s2 * inv_k - m * m, 0.0f);
      const float rstd = 1.0f / sqrtf(var + tail.eps);
      const float Gn = merged(T, jj), Bn = merged(T + 1, jj);
      v = rstd * (v - m * Gn) + Bn;
      if (gateup) u = rstd * (u - m * merged(T, jj + 8)) + merged(T + 1, jj + 8);
    }
    if (gateup) {
      v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;
    } else {
      if (tail.act == 1) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
      if (tail.res) v += elem(o == tid ? res0 : reinterpret_cast<const uint16_t*>(tail.res)[(long)t * N + n], xbf);
      if (tail.add) v += elem(o == tid ? add0 : reinterpret_cast<const uint16_t*>(tail.add)[n], xbf);
    }
    store_y(tail.y, tail.y_dtype, (long)t * N + n, v);
  }
}

}  // namespace s8
}  // namespace qlin

namespace qlin {
namespace s8 {

// Launch of one instantiation (the caller has checked the shape against it).
template <int BITS, bool LN, int MT, int GWM, int R, int W, bool XBF>
hipError_t launch_one(const S8Launch& a, hipStream_t s) {
  const Tail tail{a.y, a.res, a.add, a.eps, a.y_dtype, a.act};
  auto tp = [](const void* p, uint32_t v) { return reinterpret_cast<const void*>(tag(p, v)); };
  hipLaunchKernelGGL((s8_kernel<BITS, LN, MT, GWM, R, W, XBF>), dim3(a.grid), dim3(a.waves * 64), 0, s,
                     tp(a.x, (uint32_t)(a.K / 64) | ((uint32_t)a.x_bf16 << 15)),
                     tp(a.w0, (uint32_t)(a.T - 1) | ((uint32_t)a.gateup << 5)), tp(a.s0, (uint32_t)a.N & 0xFFFFu),
                     tp(a.b0, (uint32_t)a.N >> 16), tp(a.p1, (uint32_t)a.grid), a.p2, a.p3, tail);
  return hipGetLastError();
}

// One tile per workgroup: no ring (a second slot would only carry zeros), and up to 16
// waves where the shape has that instantiation; more tiles: two slots, up to 8 waves.
template <int BITS, bool LN, int MT, int GWM, bool XBF>
hipError_t launch_d(const S8Launch& a, hipStream_t s) {
  if (a.waves > 8) {
    if constexpr (wide_ok(BITS, LN, MT, GWM)) {
      if (a.D == 1) return launch_one<BITS, LN, MT, GWM, 1, 16, XBF>(a, s);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (max_tiles(BITS, LN, MT, GWM) >= 1) {
    if (a.D == 1) return launch_one<BITS, LN, MT, GWM, 1, 8, XBF>(a, s);
  }
  if constexpr (max_tiles(BITS, LN, MT, GWM) >= 2) {
    if (a.D <= max_tiles(BITS, LN, MT, GWM)) return launch_one<BITS, LN, MT, GWM, 2, 8, XBF>(a, s);
  }
  return hipErrorInvalidValue;
}

// One instantiation unit per (code width, LayerNorm, activation dtype), so that they compile
// in parallel; a launch whose x_bf16 does not match XBF is refused.
template <int BITS, bool LN, bool XBF>
hipError_t launch_bits_ln(const S8Launch& a, hipStream_t s) {
  if ((a.x_bf16 != 0) != XBF) return hipErrorInvalidValue;
  switch (a.MT * 100 + a.GWM) {
    case 102: return launch_d<BITS, LN, 1, 2, XBF>(a, s);
    case 104: return launch_d<BITS, LN, 1, 4, XBF>(a, s);
    case 108: return launch_d<BITS, LN, 1, 8, XBF>(a, s);
    case 116: return launch_d<BITS, LN, 1, 16, XBF>(a, s);
    case 132: return launch_d<BITS, LN, 1, 32, XBF>(a, s);
    case 202: return launch_d<BITS, LN, 2, 2, XBF>(a, s);
    case 204: return launch_d<BITS, LN, 2, 4, XBF>(a, s);
    case 208: return launch_d<BITS, LN, 2, 8, XBF>(a, s);
    case 302: return launch_d<BITS, LN, 3, 2, XBF>(a, s);
    case 304: return launch_d<BITS, LN, 3, 4, XBF>(a, s);
    case 902: return launch_d<BITS, LN, 9, 2, XBF>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace s8
}  // namespace qlin
