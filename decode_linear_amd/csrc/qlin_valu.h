// The streaming fused linear on the vector ALUs, for a few activation rows (T <= 4): the
// plain-FMA counterpart of the int8 matrix-core kernel (qlin_s8.h), built to measure where
// the matrix cores pay.  Shared by qlin_valu_q4.hip, qlin_valu_q8.hip and qlin_valu_f16.hip
// (dense fp16 weights and activations: the weight pairs go to v_dot2 as they are).
//
// Same operation and conventions as qlin_s8.h ([p1] maya-mac `_linear_kernel`: LayerNorm
// folded into the weight stream with statistics shifted by x[t, 0]; [p3] mlx-bun 0.0.10 ->
// 0.0.12 fused-decode-kernel.ts: the scale factored out of each group's dot product,
// sum_k (s q_k + b) a_k = s sum_k q_k a_k + b sum_k a_k), mapped differently:
//   * Lane (r, l) of a wave: l = lane mod LPR picks a 16-code slice of the wave's window of
//     K (LPR * 16 codes, LPR = 16 or 32), r = lane / LPR one of 64 / LPR weight rows per
//     load.  Every lane keeps its slice of each operand row (activations; with LayerNorm
//     also gamma and beta) in registers, as fp16 pairs, for the whole launch: no LDS
//     traffic per weight byte.
//   * Each operand row is scaled per wave by a power of two that puts its window's max |a|
//     in [2^14, 2^15), so fp16 holds bf16 and fp16 values exactly; the LayerNorm values
//     (x - x[t, 0]) gamma take two fp16 terms (hi + lo, 22 significant bits).
//   * Codes become exact fp16 values (a magic-number or and one packed half subtract per
//     pair), and v_dot2_f32_f16 takes two products per instruction into an fp32 sum: each
//     decoded pair serves every operand row.
//   * Per load and operand row the group's scale and bias apply once; the tile's partial
//     sums are reduced over the row's LPR lanes with DPP and row swaps, unscaled, written to
//     LDS, and merged over the waves in wave order after one barrier, followed by the same
//     LayerNorm fold and epilogue as the int8 kernel.  Deterministic, no atomics.
#pragma once

#include "qlin_s8.h"

namespace qlin {
namespace va {

using s8::elem;
using s8::gaddr;
using s8::store_y;
using s8::Tail;
using s8::tag_of;
using s8::u2_t;
using s8::u4_t;
using s8::untag;
using s8::widen8;
using s8::zaddr;
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int log2c(int v) { return v <= 1 ? 0 : 1 + log2c(v / 2); }

template <int BITS, bool LN, int TT, int LPR>
struct VCfg {
  static constexpr int CPL = 16;                   // codes per lane and load
  static constexpr int CB = CPL * BITS / 8;        // their bytes (8, 16, or 32 for dense fp16)
  static constexpr int LB = log2c(LPR);
  static constexpr int KW = LPR * CPL;             // k of one wave's window
  static constexpr int RPL = 64 / LPR;             // weight rows per load
  static constexpr int NL = 16 / RPL;              // loads per 16-row tile
  static constexpr int OR = TT + (LN ? 2 : 0);     // operand rows (gamma, beta last)
  static constexpr int NTX = LN ? 2 : 1;           // fp16 terms of an activation row
  static constexpr int PAIRS = CPL / 2;            // fp16 pairs of a slice
  static constexpr int WMAX = 16;                  // waves of a workgroup at most
  static constexpr int PMAX = 8;                   // tiles of a workgroup at most
  static constexpr int PART_FLOATS = PMAX * WMAX * 16 * OR;
  static constexpr int ST_FLOATS = WMAX * TT * 2;
  static_assert(LPR == 16 || LPR == 32, "16 or 32 lanes per weight row");
  static constexpr int MAXW = (LPR == 16 && !LN) ? 16 : 8;   // waves of a launch at most (VGPR budget)
  static_assert(TT >= 1 && TT <= 4, "up to four activation rows");
};

__device__ __forceinline__ uint32_t h2_bits(h2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2_t bits_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// fp16 pair (1024 + c0, 1024 + c1) from two code fields at bits 0 and 16 of w (masked),
// minus 1024: the exact codes.
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t mask) {
  return h2_bits(bits_h2((w & mask) | 0x64006400u) - (h2_t){(_Float16)1024.0f, (_Float16)1024.0f});
}

// The slice's codes as PAIRS fp16 pairs (dense fp16 weights: the elements as they are); pair
// order below matches the activation pairs built in staging (pair_k).
template <int BITS> __device__ __forceinline__ void decode(const uint32_t* w, uint32_t* cp) {
  if constexpr (BITS == 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) cp[i] = w[i];   // elements 2i, 2i+1
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int m = 0; m < 4; ++m) cp[4 * d + m] = code_pair(w[d] >> (4 * m), 0x000F000Fu);   // codes 8d+m, 8d+m+4
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      cp[2 * d] = code_pair(w[d], 0x00FF00FFu);              // codes 4d, 4d+2
      cp[2 * d + 1] = code_pair(w[d] >> 8, 0x00FF00FFu);     // codes 4d+1, 4d+3
    }
  }
}
// Slice positions of the two elements of pair i.
template <int BITS> __device__ __forceinline__ constexpr int pair_k(int i, int h) {
  return BITS == 16 ? 2 * i + h : BITS == 4 ? 8 * (i >> 2) + (i & 3) + 4 * h : 4 * (i >> 1) + (i & 1) + 2 * h;
}

// Sum over lane bits [0, LB) in a fixed order (xor 1, 2, 4, 8, 16, 32), the same value on
// every lane of the group: DPP quad permutes, a row shift pair, a row rotation, row swaps.
template <int CTRL> __device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int LB> __device__ __forceinline__ float slice_sum(float v) {
  if constexpr (LB >= 1) v += dppf<0xB1>(v);
  if constexpr (LB >= 2) v += dppf<0x4E>(v);
  if constexpr (LB >= 3) {
    const float dn = dppf<0x114>(v), up = dppf<0x104>(v);
    v += (threadIdx.x & 4) ? dn : up;
  }
  if constexpr (LB >= 4) v += dppf<0x128>(v);
  if constexpr (LB >= 5) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    v = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
  }
  if constexpr (LB >= 6) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    v = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
  }
  return v;
}

// Window exponent of an operand row from the bits of its max |a|: max * 2^e in [2^14, 2^15);
// 0 for a zero row, clamped so that 2^-e stays a normal float.
__device__ __forceinline__ int wexp(uint32_t amax_bits) {
  if (amax_bits == 0u) return 0;
  const int e = 14 - ((int)(amax_bits >> 23) - 127);
  return e > 100 ? 100 : e;
}

template <int BITS, bool LN, int TT, int LPR>
__global__ __attribute__((amdgpu_flat_work_group_size(1, VCfg<BITS, LN, TT, LPR>::MAXW * 64))) void valu_kernel(
    const void* xt, const void* w0t, const void* s0t, const void* b0t, const void* p1t, const void* p2t,
    const void* p3t, const Tail tail) {
  using C = VCfg<BITS, LN, TT, LPR>;
  __shared__ __attribute__((aligned(16))) float parts[C::PART_FLOATS];
  __shared__ float sts[C::ST_FLOATS];

  const uint32_t tx = tag_of(xt), tw = tag_of(w0t);
  const int G = (int)(tx & 0x7FFFu), K = G << 6;
  const bool xbf = (tx >> 15) != 0;
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
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int waves = (K + C::KW - 1) / C::KW;
  const int sl = lane & (LPR - 1), rs = lane >> C::LB;   // slice, row slot
  const int k0 = wv * C::KW + sl * C::CPL;                // first k of this lane's slice
  const bool kin = k0 < K;
  const int grp = k0 >> 6;                                 // its quantization group
  const int ntw = (ntiles - (int)blockIdx.x + grid - 1) / grid;   // tiles of this workgroup

  // ---- tile loads: a ring of two slots, each the NL loads of one tile ----------------------
  struct Slot {
    uint32_t code[C::NL][C::CB / 4];
    uint32_t sb[C::NL];   // scale | bias << 16
  };
  auto issue = [&](Slot& r, int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int l = 0; l < C::NL; ++l) {
      const int jr = rs + C::RPL * l;   // weight row of the tile
      int proj, n;
      if (gateup) { proj = jr >> 3; n = tile * 8 + (jr & 7); }
      else { proj = 0; n = tile * 16 + jr; }
      const bool ok = kin && tile < ntiles && n < N;
      const void* wb = proj ? p1 : (const void*)w0;
      const long off = (long)n * row_bytes + (long)k0 * BITS / 8;
      if constexpr (C::CB == 32) {
        const u4_t v0 = *(ok ? gaddr<u4_t>(wb, off) : zaddr<u4_t>(0));
        const u4_t v1 = *(ok ? gaddr<u4_t>(wb, off + 16) : zaddr<u4_t>(0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r.code[l][i] = v0[i];
          r.code[l][4 + i] = v1[i];
        }
      } else if constexpr (C::CB == 16) {
        const u4_t v = *(ok ? gaddr<u4_t>(wb, off) : zaddr<u4_t>(0));
#pragma unroll
        for (int i = 0; i < 4; ++i) r.code[l][i] = v[i];
      } else {
        const u2_t v = *(ok ? gaddr<u2_t>(wb, off) : zaddr<u2_t>(0));
        r.code[l][0] = v[0];
        r.code[l][1] = v[1];
      }
      if constexpr (BITS == 16) {
        r.sb[l] = 0x3C00u;   // dense: scale 1, bias 0
      } else {
        const void* sp = proj ? p2 : (const void*)s0;
        const void* bp = proj ? p3 : (const void*)b0;
        const long so = ((long)n * G + grp) * 2;
        const uint32_t sv = *(ok ? gaddr<uint16_t>(sp, so) : zaddr<uint16_t>(0));
        const uint32_t bv = *(ok ? gaddr<uint16_t>(bp, so) : zaddr<uint16_t>(0));
        r.sb[l] = sv | (bv << 16);
      }
    }
  };
  Slot ring[2];
  const int nq = (ntw + 1) & ~1;   // steps: a multiple of two; steps past ntw carry zeros
  auto tile_of = [&](int q) __attribute__((always_inline)) { return q < ntw ? (int)blockIdx.x + q * grid : ntiles; };
  issue(ring[0], tile_of(0));
  issue(ring[1], tile_of(1));

  // ---- staging: this lane's slice of every operand row, as fp16 pairs -------------------------
  const uint16_t* gam = LN ? static_cast<const uint16_t*>(p1) : nullptr;
  const uint16_t* bet = LN ? static_cast<const uint16_t*>(p2) : nullptr;
  auto load16 = [&](const uint16_t* base, long elem_off, bool ok, float v[16]) __attribute__((always_inline)) {
    const u4_t a = *(ok ? gaddr<u4_t>(base, elem_off * 2) : zaddr<u4_t>(0));
    const u4_t b = *(ok ? gaddr<u4_t>(base, elem_off * 2 + 16) : zaddr<u4_t>(0));
    widen8(a, xbf, v);
    widen8(b, xbf, v + 8);
  };
  uint32_t xa[TT][C::NTX][C::PAIRS];   // activation rows (LN: (x - x0) gamma in two terms)
  uint32_t xgb[LN ? 2 : 1][C::PAIRS];  // LN: gamma and beta
  float xs[C::OR];                      // sum of the lane's slice of each operand row, as staged
  float unit[C::OR];                    // 2^-e of each operand row
  bool poison[C::OR];
  float gv[16], bv[16];
  if constexpr (LN) {
    load16(gam, k0, kin, gv);
    load16(bet, k0, kin, bv);
  }
  // one operand row: window max over the slices, the scale, the fp16 terms and their sum
  auto stage_row = [&](const float v[16], uint32_t (*out)[C::PAIRS], int nterm, float& sum, float& un,
                       bool& bad) __attribute__((always_inline)) {
    uint32_t m = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = max(m, __builtin_bit_cast(uint32_t, v[e]) & 0x7FFFFFFFu);
    m = s8::group_max<LPR>(m);
    bad = (m >> 23) >= 255u;
    const int ex = wexp(m);
    un = __builtin_bit_cast(float, (uint32_t)(127 - ex) << 23);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < C::PAIRS; ++i) {
      float hv[2], lv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float a = __builtin_amdgcn_ldexpf(v[pair_k<BITS>(i, h)], ex);
        const _Float16 hi = (_Float16)a;
        hv[h] = (float)hi;
        lv[h] = a - hv[h];
      }
      out[0][i] = h2_bits((h2_t){(_Float16)hv[0], (_Float16)hv[1]});
      s += hv[0] + hv[1];
      if (nterm > 1) {
        const h2_t lo = (h2_t){(_Float16)lv[0], (_Float16)lv[1]};
        out[1][i] = h2_bits(lo);
        s += (float)lo[0] + (float)lo[1];
      }
    }
    sum = s;
  };
  float st1[TT], st2[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float v[16];
    const bool rin = t < T;
    load16(x, (long)t * K + k0, kin && rin, v);
    float s1 = 0.0f, s2 = 0.0f;
    if constexpr (LN) {
      const float x0 = elem(*(rin ? gaddr<uint16_t>(x, (long)t * K * 2) : zaddr<uint16_t>(0)), xbf);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float d = (kin && rin) ? v[e] - x0 : 0.0f;
        s1 += d;
        s2 = fmaf(d, d, s2);
        v[e] = d * gv[e];
      }
    }
    st1[t] = s1;
    st2[t] = s2;
    stage_row(v, xa[t], C::NTX, xs[t], unit[t], poison[t]);
  }
  if constexpr (LN) {
    stage_row(gv, &xgb[0], 1, xs[TT], unit[TT], poison[TT]);
    stage_row(bv, &xgb[1], 1, xs[TT + 1], unit[TT + 1], poison[TT + 1]);
  }
  if constexpr (LN) {   // the window's shifted sums of each row, for the statistics
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float a = slice_sum<C::LB>(st1[t]), b = slice_sum<C::LB>(st2[t]);
      if (lane == 0) {
        sts[(wv * TT + t) * 2] = a;
        sts[(wv * TT + t) * 2 + 1] = b;
      }
    }
  }

  // ---- the tiles ---------------------------------------------------------------------------
  // per load: the slice's dot products with every operand row, the group's scale and bias,
  // the sum over the row's LPR lanes; lane 0 of each row slot writes the tile's partials
  auto compute = [&](const Slot& r, int i, bool keep) __attribute__((always_inline)) {
#pragma unroll
    for (int l = 0; l < C::NL; ++l) {
      uint32_t cp[C::PAIRS];
      decode<BITS>(r.code[l], cp);
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.sb[l] & 0xFFFFu));
      const float b = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.sb[l] >> 16));
#pragma unroll
      for (int t = 0; t < C::OR; ++t) {
        float d = 0.0f;
#pragma unroll
        for (int q = 0; q < C::PAIRS; ++q) {
          if (t < TT) {
#pragma unroll
            for (int h = 0; h < C::NTX; ++h) d = __builtin_amdgcn_fdot2(bits_h2(cp[q]), bits_h2(xa[t < TT ? t : 0][h][q]), d, false);
          } else {
            d = __builtin_amdgcn_fdot2(bits_h2(cp[q]), bits_h2(xgb[LN ? t - TT : 0][q]), d, false);
          }
        }
        const float v = slice_sum<C::LB>(fmaf(s, d, b * xs[t]));
        if (keep && sl == 0)
          parts[((i * C::WMAX + wv) * 16 + rs + C::RPL * l) * C::OR + t] = poison[t] ? __builtin_nanf("") : v * unit[t];
      }
    }
  };
  for (int q0 = 0; q0 < nq; q0 += 2) {
    compute(ring[0], q0, q0 < ntw);
    issue(ring[0], tile_of(q0 + 2));
    compute(ring[1], q0 + 1, q0 + 1 < ntw);
    issue(ring[1], tile_of(q0 + 3));
  }

  // ---- merge over the waves, LayerNorm fold, epilogue, store ---------------------------------
  __syncthreads();
  const int nthreads = waves * 64;
  const int per_tile = gateup ? 8 * T : 16 * T;
  const float inv_k = 1.0f / (float)K;
  for (int o = tid; o < ntw * per_tile; o += nthreads) {
    const int i = o / per_tile, rem = o - i * per_tile;
    const int t = gateup ? rem >> 3 : rem >> 4, jj = gateup ? rem & 7 : rem & 15;
    const int tile = (int)blockIdx.x + i * grid;
    const int n = gateup ? tile * 8 + jj : tile * 16 + jj;
    if (n >= N) continue;
    auto merged = [&](int orow, int col) __attribute__((always_inline)) {
      float v = 0.0f;
      for (int w = 0; w < waves; ++w) v += parts[((i * C::WMAX + w) * 16 + col) * C::OR + orow];
      return v;
    };
    float v = merged(t, jj);
    float u = gateup ? merged(t, jj + 8) : 0.0f;
    if constexpr (LN) {
      float s1 = 0.0f, s2 = 0.0f;
      for (int w = 0; w < waves; ++w) {
        s1 += sts[(w * TT + t) * 2];
        s2 += sts[(w * TT + t) * 2 + 1];
      }
      const float m = s1 * inv_k;
      const float var = fmaxf(s2 * inv_k - m * m, 0.0f);
      const float rstd = 1.0f / sqrtf(var + tail.eps);
      v = rstd * (v - m * merged(TT, jj)) + merged(TT + 1, jj);
      if (gateup) u = rstd * (u - m * merged(TT, jj + 8)) + merged(TT + 1, jj + 8);
    }
    if (gateup) {
      v = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * u;
    } else {
      if (tail.act == 1) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
      if (tail.res) v += elem(reinterpret_cast<const uint16_t*>(tail.res)[(long)t * N + n], xbf);
      if (tail.add) v += elem(reinterpret_cast<const uint16_t*>(tail.add)[n], xbf);
    }
    store_y(tail.y, tail.y_dtype, (long)t * N + n, v);
  }
}

// Launch of one instantiation (the caller has checked the shape against it).
template <int BITS, bool LN, int TT, int LPR>
hipError_t launch_one(const S8Launch& a, hipStream_t s) {
  const Tail tail{a.y, a.res, a.add, a.eps, a.y_dtype, a.act};
  auto tp = [](const void* p, uint32_t v) { return reinterpret_cast<const void*>(s8::tag(p, v)); };
  hipLaunchKernelGGL((valu_kernel<BITS, LN, TT, LPR>), dim3(a.grid), dim3(a.waves * 64), 0, s,
                     tp(a.x, (uint32_t)(a.K / 64) | ((uint32_t)a.x_bf16 << 15)),
                     tp(a.w0, (uint32_t)(a.T - 1) | ((uint32_t)a.gateup << 5)), tp(a.s0, (uint32_t)a.N & 0xFFFFu),
                     tp(a.b0, (uint32_t)a.N >> 16), tp(a.p1, (uint32_t)a.grid), a.p2, a.p3, tail);
  return hipGetLastError();
}

// a.MT carries the activation rows the instantiation holds (1, 2 or 4), a.GWM the lanes per
// weight row (16: up to 16 waves; 32: up to 8).
template <int BITS, bool LN>
hipError_t launch_bits_ln(const S8Launch& a, hipStream_t s) {
  switch (a.MT * 100 + a.GWM) {
    case 116: return launch_one<BITS, LN, 1, 16>(a, s);
    case 132: return launch_one<BITS, LN, 1, 32>(a, s);
    case 216: return launch_one<BITS, LN, 2, 16>(a, s);
    case 232: return launch_one<BITS, LN, 2, 32>(a, s);
    case 416: return launch_one<BITS, LN, 4, 16>(a, s);
    case 432:   // with LayerNorm this one would spill registers: not instantiated
      if constexpr (!LN) return launch_one<BITS, LN, 4, 32>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace va
}  // namespace qlin
