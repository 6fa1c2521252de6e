// attend for gfx950: one pass of a decoder layer's attention over a short band of
// positions ([p1] maya-mac src/maya_mac/mlx_kernels.py, `_ATTEND` and `attend()`).
//
//   kv_out (2, H, P + T, HD) = the cached keys / values (2, H, P, HD), then this pass's
//                              T rows taken from qkv (bit patterns copied)
//   out[t, h*HD + d]         = sum_{j <= P + t} p_j v_j[d],
//       p_j = softmax_j(s),  s_j = (q_t . k_j) / sqrt(HD)      (causal, fp32 throughout)
//
// qkv (T, 3D), D = H * HD, holds per new position the query, key and value of every head
// (columns [0, D), [D, 2D), [2D, 3D); head h owns HD consecutive columns of each).
//
// Mapping (wave64): one wave per (head, new position).  Lane l scores key j = l mod 32
// over half l / 32 of the head dimensions, with 16-byte loads; one lane swap adds the two
// halves, so lanes j and j + 32 hold the same score.  The softmax max and sum are
// butterflies over the wave; the weighted value sum runs with lanes over head dimensions
// (coalesced rows of v) and the weights broadcast from their key lanes.  The cache copy is
// spread over the T waves of a head.  Nothing is staged in LDS: every row is read once per
// wave from L2, and each phase issues its loads together (clamped to valid rows, the extra
// ones masked) so that a wave waits for one round of loads per phase, not one per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_internal.h"

namespace qlin {
namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
constexpr int kAttendKeys = 32;   // visible keys at most (cached + new positions)

__device__ __forceinline__ float bits_to_float(uint32_t h, int dtype) {
  if (dtype == 2) return __builtin_bit_cast(float, h << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// The 16-bit halves of a 16-byte piece as floats.
__device__ __forceinline__ void widen8(const u4_t v, int dtype, float f[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bits_to_float(v[i] & 0xFFFFu, dtype);
    f[2 * i + 1] = bits_to_float(v[i] >> 16, dtype);
  }
}

// Butterflies over the wave without LDS: v op v[lane ^ 2^B] for B = 0 .. 5 (DPP quad
// permutes, a row shift pair, a row rotation, then the gfx950 row swaps, which return both
// rows of a pair); op is commutative, so both lanes of every pair get the same value.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <bool MAX> __device__ __forceinline__ float wave_all(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_f<0xB1>(v));                                     // xor 1
  v = op(v, dpp_f<0x4E>(v));                                     // xor 2
  {
    const float dn = dpp_f<0x114>(v), up = dpp_f<0x104>(v);      // row_shr:4, row_shl:4
    v = op(v, (threadIdx.x & 4) ? dn : up);                      // xor 4
  }
  v = op(v, dpp_f<0x128>(v));                                    // row_ror:8: xor 8
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    v = op(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));   // xor 16
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    v = op(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));   // xor 32
  }
  return v;
}
__device__ __forceinline__ float wave_max(float v) { return wave_all<true>(v); }
__device__ __forceinline__ float wave_sum(float v) { return wave_all<false>(v); }
// The value of the lane across the halves (lane ^ 32).
__device__ __forceinline__ float other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, (int)((threadIdx.x & 32) ? r[0] : r[1]));
}

// One RNE rounding of an fp32 value to the output dtype.
__device__ __forceinline__ void store_elem(void* y, int dtype, long idx, float v) {
  if (dtype == 0) {
    static_cast<float*>(y)[idx] = v;
  } else if (dtype == 1) {
    static_cast<_Float16*>(y)[idx] = (_Float16)v;
  } else {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    uint16_t r;
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) r = (uint16_t)((b >> 16) | 0x40u);   // quiet NaN
    else r = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
    static_cast<uint16_t*>(y)[idx] = r;
  }
}

// DT, the dtype of qkv and kv (1 fp16, 2 bf16), is part of the instantiation: as a runtime
// flag every element was widened both ways and one result selected (6.49 -> 5.41 us on the
// 16-head, 24 + 8 position band).
template <int DT>
__global__ __launch_bounds__(64) void attend_kernel(const AttendParams a) {
  const int h = blockIdx.x, t = blockIdx.y, lane = threadIdx.x;
  const int H = a.H, HD = a.HD, P = a.P, T = a.T;
  const long D = (long)H * HD, L = P + T;
  const int pieces = HD / 8;   // 16-byte pieces per row
  const uint16_t* qkv = static_cast<const uint16_t*>(a.qkv);
  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  uint16_t* kv_out = static_cast<uint16_t*>(a.kv_out);

  // The cache: this wave's new rows (position P + t), and the cached rows j = t, t + T, ...
  // Four pieces per lane are loaded before any is stored.
  const int mine = P > t ? (P - t + T - 1) / T : 0;
  const int items = (1 + mine) * 2 * pieces;
  for (int i0 = lane; i0 < items; i0 += 4 * 64) {
    u4_t buf[4];
    long dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(i0 + 64 * u, items - 1);
      const int r = i / (2 * pieces), kvsel = (i / pieces) & 1, pc = i % pieces;
      const long j = r == 0 ? (long)(P + t) : t + (long)(r - 1) * T;
      const u4_t* src = r == 0 ? reinterpret_cast<const u4_t*>(qkv + (long)t * 3 * D + (1 + kvsel) * D + (long)h * HD) + pc
                               : reinterpret_cast<const u4_t*>(kv + (((long)kvsel * H + h) * P + j) * HD) + pc;
      buf[u] = *src;
      dst[u] = (((long)kvsel * H + h) * L + j) * HD / 8 + pc;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + 64 * u < items) reinterpret_cast<u4_t*>(kv_out)[dst[u]] = buf[u];
  }
  if (a.last && t != T - 1) return;

  // Scores: lane (j, half) takes key j over half of the head dimensions; the pieces of a
  // batch of four are loaded before their products (keys past pos read key pos, masked).
  const int pos = P + t;   // keys 0 .. pos are visible
  const int j = lane & 31, half = lane >> 5;
  const int jk = min(j, pos);
  const uint16_t* krow = jk < P ? kv + ((long)h * P + jk) * HD : qkv + (long)(jk - P) * 3 * D + D + (long)h * HD;
  const u4_t* q4 = reinterpret_cast<const u4_t*>(qkv + (long)t * 3 * D + (long)h * HD);
  const u4_t* k4 = reinterpret_cast<const u4_t*>(krow);
  const int hp = pieces / 2, pc_lo = half * hp;
  float dot = 0.0f;
  for (int b = 0; b < hp; b += 4) {
    u4_t qw[4], kw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = pc_lo + min(b + u, hp - 1);
      qw[u] = q4[pc];
      kw[u] = k4[pc];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (b + u >= hp) break;
      float qf[8], kf[8];
      widen8(qw[u], DT, qf);
      widen8(kw[u], DT, kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qf[e], kf[e], dot);
    }
  }
  // lanes j and j + 32 swap halves: both hold the key's whole dot product, in one order
  const float other = other_half(dot);
  const float full = half == 0 ? dot + other : other + dot;
  const float s = j <= pos ? full * a.scale : -__builtin_inff();
  const float m = wave_max(s);
  const float e = j <= pos ? expf(s - m) : 0.0f;
  const float z = wave_sum(half == 0 ? e : 0.0f);
  const float p = e / z;

  // Values: lanes over head dimensions; every visible row's element is loaded before the
  // sum, which runs over the keys in order with each weight read from its key's lane.
  const long row = a.last ? 0 : t;
  for (int d = lane; d < HD; d += 64) {
    uint32_t vv[kAttendKeys];   // bit patterns, widened at their use
#pragma unroll
    for (int jj = 0; jj < kAttendKeys; ++jj) {
      const int jc = min(jj, pos);
      const uint16_t* vrow = jc < P ? kv + (((long)H + h) * P + jc) * HD : qkv + (long)(jc - P) * 3 * D + 2 * D + (long)h * HD;
      vv[jj] = vrow[d];
    }
    __builtin_amdgcn_sched_barrier(0);
    float o = 0.0f;
#pragma unroll
    for (int jj = 0; jj < kAttendKeys; ++jj) {
      const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), jj));
      o = jj <= pos ? fmaf(pj, bits_to_float(vv[jj], DT), o) : o;
    }
    store_elem(a.out, a.out_dtype, row * D + (long)h * HD + d, o);
  }
}

}  // namespace

hipError_t launch_attend(const AttendParams& a, hipStream_t s) {
  if (a.dtype == 1) hipLaunchKernelGGL(attend_kernel<1>, dim3(a.H, a.T), dim3(64), 0, s, a);
  else hipLaunchKernelGGL(attend_kernel<2>, dim3(a.H, a.T), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlin
