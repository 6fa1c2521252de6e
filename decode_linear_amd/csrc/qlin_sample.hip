// One sampling step of the depth decoder for gfx950 ([p1] maya-mac src/maya_mac/mlx_kernels.py,
// the sampling kernel and `sample()`): keep the top_k largest logits (every logit equal to the
// top_k-th stays), pick one of them by Gumbel-max, and append the picked code's embedding row.
//
//   rank(f)   order-preserving 32-bit image of the fp32 logit f (larger logit, larger rank;
//             -0 ranks below +0): the bits of f with the sign flipped, all bits flipped for
//             negative f
//   theta     the top_k-th largest rank: exact, by a most-significant-digit-first radix
//             select over 8-bit digits
//   code      among the codes with rank >= theta, the one with the largest score
//             fl32(fl32(f * inv_temp) + gumbel), the smaller index among equal scores (+0
//             and -0 are equal); NaN scores never win; -1 when no kept score is a number
//   out       the prefix rows, then (with a table) the code's row of the table (zeros for -1)
//
// Mapping: one workgroup of 256 threads; thread t keeps the ranks of codes t, t + 256, ... in
// registers (PER of them: 8, 16 or 32, the fewest that hold n <= 8192).  Radix pass: each
// wave counts the digits of its matching ranks into its own 256-bin LDS histogram (LDS
// integer atomics, private to the wave), then all 256 threads take one digit each, highest
// digit first, add the four waves' counts and run one prefix sum over the workgroup; the
// thread whose digit holds the wanted rank publishes it.
// Gumbel-max: every candidate becomes one 64-bit word, (rank of the score) << 32 | ~index, so
// the winner is the plain maximum of the words (an exact, order-free reduction: the result
// does not depend on the order of the combines).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_internal.h"

namespace qlin {
namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
constexpr int kThr = 256;                     // threads of the workgroup
constexpr int kWv = kThr / 64;                // its waves
constexpr int kPerMax = kSampleMaxCodes / kThr;  // ranks per thread, at most

__device__ __forceinline__ uint32_t rank_of(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u >> 31) ? ~u : (u ^ 0x80000000u);
}
__device__ __forceinline__ float logit_of(uint32_t r) {
  return __builtin_bit_cast(float, (r >> 31) ? (r ^ 0x80000000u) : ~r);
}
// The bits of logit i (LD: 0 fp32, 1 fp16, 2 bf16) and their exact fp32 value.
template <int LD> __device__ __forceinline__ uint32_t logit_bits(const void* logits, int i) {
  if constexpr (LD == 0) return static_cast<const uint32_t*>(logits)[i];
  else return static_cast<const uint16_t*>(logits)[i];
}
template <int LD> __device__ __forceinline__ float logit_value(uint32_t b) {
  if constexpr (LD == 0) return __builtin_bit_cast(float, b);
  else if constexpr (LD == 1) return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  else return __builtin_bit_cast(float, b << 16);
}
// Candidate word of code i with score s: 0 (never wins) for a NaN score; otherwise the rank of
// s (with -0 taken as +0) above the complement of i, so that a larger score, then a smaller
// index, gives a larger word.
__device__ __forceinline__ uint64_t candidate(float s, uint32_t i) {
  if (s != s) return 0ull;
  const uint32_t r = rank_of(s == 0.0f ? 0.0f : s);
  return ((uint64_t)r << 32) | (uint64_t)(~i);
}

template <int CTRL> __device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  // lanes whose source is outside the row read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t lane_u(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
// Inclusive prefix sum over the 64 lanes (lane l: sum of lanes 0..l): a scan within each
// 16-lane row by DPP row shifts (1, 2, 4, 8), then each row adds the totals of the rows
// before it, read from their last lanes (no LDS round trip).
__device__ __forceinline__ uint32_t wave_prefix(uint32_t v, int lane) {
  v += dpp_u<0x111>(v);   // row_shr:1
  v += dpp_u<0x112>(v);   // row_shr:2
  v += dpp_u<0x114>(v);   // row_shr:4
  v += dpp_u<0x118>(v);   // row_shr:8
  const uint32_t r0 = lane_u(v, 15), r1 = lane_u(v, 31), r2 = lane_u(v, 47);
  return v + (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
}
// Maximum of a 64-bit word over the wave (every lane ends with it): butterflies within each
// 16-lane row (xor 1, 2, 4, 8 by DPP), then the four rows' maxima read from lanes 0, 16, 32
// and 48.  A maximum is exact in any order.
__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL> __device__ __forceinline__ uint64_t dpp64(uint64_t w) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(w >> 32), CTRL, 0xF, 0xF, false);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)w, CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max64(uint64_t w, int lane) {
  w = max64(w, dpp64<0xB1>(w));   // quad_perm [1, 0, 3, 2]: xor 1
  w = max64(w, dpp64<0x4E>(w));   // quad_perm [2, 3, 0, 1]: xor 2
  {
    const uint64_t dn = dpp64<0x114>(w), up = dpp64<0x104>(w);   // row_shr:4, row_shl:4
    w = max64(w, (lane & 4) ? dn : up);                          // xor 4
  }
  w = max64(w, dpp64<0x128>(w));  // row_ror:8: xor 8
  const uint32_t hi = (uint32_t)(w >> 32), lo = (uint32_t)w;
  uint64_t m = ((uint64_t)lane_u(hi, 0) << 32) | lane_u(lo, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) m = max64(m, ((uint64_t)lane_u(hi, 16 * r) << 32) | lane_u(lo, 16 * r));
  return m;
}

template <int LD, int PER>
__global__ __launch_bounds__(kThr) void sample_kernel(const SampleParams a) {
#pragma clang fp contract(off)
  static_assert(PER >= 1 && PER <= kPerMax, "ranks per thread");
  __shared__ uint32_t counts[kWv][256];   // one digit histogram per wave
  __shared__ uint32_t wave_total[kWv];
  __shared__ uint32_t sel_digits, sel_left;   // the selected high digits, and ranks still wanted
  __shared__ uint64_t wave_best[kWv];
  __shared__ int32_t picked;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int n = a.n;
  const long pieces = (long)a.D * a.es / 16;   // 16-byte pieces of one row
  u4_t* out = static_cast<u4_t*>(a.out);

  // The prefix rows do not depend on the code: their copy goes out first, eight pieces in
  // flight per thread, under the selection.
  if (a.copy_prefix) {
    const u4_t* src = static_cast<const u4_t*>(a.prefix);
    const long total = (long)a.n_prev * pieces;
    long p = t;
    for (; p + 7L * kThr < total; p += 8L * kThr) {
      u4_t buf[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) buf[u] = src[p + (long)u * kThr];
#pragma unroll
      for (int u = 0; u < 8; ++u) out[p + (long)u * kThr] = buf[u];
    }
    for (; p < total; p += kThr) out[p] = src[p];
  }

  // Every logit and noise value of this thread is loaded before any is used (indices past n
  // read element n - 1 and are masked), so the selection waits for one round of loads.
  uint32_t rk[PER];
  float gm[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = min(t + kThr * e, n - 1);
    rk[e] = logit_bits<LD>(a.logits, i);
    gm[e] = a.gumbel[i];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) rk[e] = t + kThr * e < n ? rank_of(logit_value<LD>(rk[e])) : 0u;

  // ---- theta: 8-bit digits, most significant first ---------------------------------------
  // A 16-bit logit widens to an fp32 value whose low mantissa bits are zero (16 of them for
  // bf16, 13 for fp16), so the rank's low digits are the same for every logit of one sign:
  // the select stops after 2 digits (bf16) or 3 (fp16) and fills the rest from the sign
  // (bf16 logits, 2048 codes: 6.62 -> 5.31 us).
  constexpr int NPASS = LD == 2 ? 2 : (LD == 1 ? 3 : 4);
  uint32_t digits = 0u, left = (uint32_t)a.top_k;   // chosen so far (uniform), ranks wanted
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    const int sh = 24 - 8 * pass;
#pragma unroll
    for (int w = 0; w < kWv; ++w) counts[w][t] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = t + kThr * e;
      const bool on_path = pass == 0 || (rk[e] >> (sh + 8)) == digits;
      if (i < n && on_path) atomicAdd(&counts[wv][(rk[e] >> sh) & 0xFFu], 1u);
    }
    __syncthreads();
    // thread t owns digit 255 - t: how many matching ranks carry it, and how many carry a
    // higher digit (a prefix sum over the threads in order)
    const uint32_t dgt = 255u - (uint32_t)t;
    uint32_t mine = 0u;
#pragma unroll
    for (int w = 0; w < kWv; ++w) mine += counts[w][dgt];
    const uint32_t incl = wave_prefix(mine, lane);
    if (lane == 63) wave_total[wv] = incl;
    __syncthreads();
    uint32_t above = incl - mine;
    for (int w = 0; w < wv; ++w) above += wave_total[w];
    if (above < left && left <= above + mine) {   // exactly one thread: its digit holds the rank
      sel_digits = (digits << 8) | dgt;
      sel_left = left - above;
    }
    __syncthreads();
    digits = sel_digits;
    left = sel_left;
  }
  // the unselected low digits: zeros under a positive logit's rank (top bit set), ones under
  // a negative one's
  constexpr int LOW = 8 * (4 - NPASS);
  const uint32_t fill = LOW == 0 ? 0u : (((digits >> (8 * NPASS - 1)) & 1u) ? 0u : (1u << LOW) - 1u);
  const uint32_t theta = LOW == 0 ? digits : ((digits << LOW) | fill);

  // ---- Gumbel-max over the kept codes ------------------------------------------------------
  uint64_t best = 0ull;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = t + kThr * e;
    if (i < n && rk[e] >= theta) {
      const float scaled = logit_of(rk[e]) * a.inv_temp;   // one fp32 rounding
      const float s = scaled + gm[e];                      // and another (no contraction)
      const uint64_t c = candidate(s, (uint32_t)i);
      best = c > best ? c : best;
    }
  }
  best = wave_max64(best, lane);
  if (lane == 0) wave_best[wv] = best;
  __syncthreads();
  if (t == 0) {
    uint64_t b = wave_best[0];
#pragma unroll
    for (int w = 1; w < kWv; ++w) b = wave_best[w] > b ? wave_best[w] : b;
    const int32_t code = b == 0ull ? -1 : (int32_t)(~(uint32_t)b);
    picked = code;
    *a.code = code;
  }
  __syncthreads();

  // ---- the picked code's embedding row after the prefix --------------------------------------
  if (a.table) {
    const int32_t code = picked;
    const u4_t* row = static_cast<const u4_t*>(a.table) + (long)(code < 0 ? 0 : code) * pieces;
    for (long p = t; p < pieces; p += kThr)
      out[(long)a.n_prev * pieces + p] = code < 0 ? (u4_t){0u, 0u, 0u, 0u} : row[p];
  }
}

// Ranks per thread: the fewest of 8, 16 and 32 that hold n (with 32 for every n, a call of
// 2048 codes ran 4 x the loads and loop trips it needed: 10.16 -> 6.65 us).
template <int LD>
void launch_ld(const SampleParams& a, hipStream_t s) {
  if (a.n <= 8 * kThr) hipLaunchKernelGGL((sample_kernel<LD, 8>), dim3(1), dim3(kThr), 0, s, a);
  else if (a.n <= 16 * kThr) hipLaunchKernelGGL((sample_kernel<LD, 16>), dim3(1), dim3(kThr), 0, s, a);
  else hipLaunchKernelGGL((sample_kernel<LD, kPerMax>), dim3(1), dim3(kThr), 0, s, a);
}

}  // namespace

hipError_t launch_sample(const SampleParams& a, hipStream_t s) {
  if (a.logit_dtype == 0) launch_ld<0>(a, s);
  else if (a.logit_dtype == 1) launch_ld<1>(a, s);
  else launch_ld<2>(a, s);
  return hipGetLastError();
}

}  // namespace qlin
