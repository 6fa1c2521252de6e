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
// wave from L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_internal.h"

namespace qlin {
namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
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

__global__ __launch_bounds__(64) void attend_kernel(const AttendParams a) {
  const int h = blockIdx.x, t = blockIdx.y, lane = threadIdx.x;
  const int H = a.H, HD = a.HD, P = a.P, T = a.T;
  const long D = (long)H * HD, L = P + T;
  const int pieces = HD / 8;   // 16-byte pieces per row
  const uint16_t* qkv = static_cast<const uint16_t*>(a.qkv);
  const uint16_t* kv = static_cast<const uint16_t*>(a.kv);
  uint16_t* kv_out = static_cast<uint16_t*>(a.kv_out);

  // The cache: this wave's new rows (position P + t), and the cached rows j = t, t + T, ...
  const int mine = P > t ? (P - t + T - 1) / T : 0;
  for (int i = lane; i < (1 + mine) * 2 * pieces; i += 64) {
    const int r = i / (2 * pieces), kvsel = (i / pieces) & 1, pc = i % pieces;
    const u4_t* src;
    long j;
    if (r == 0) {
      j = P + t;
      src = reinterpret_cast<const u4_t*>(qkv + (long)t * 3 * D + (1 + kvsel) * D + (long)h * HD) + pc;
    } else {
      j = t + (long)(r - 1) * T;
      src = reinterpret_cast<const u4_t*>(kv + (((long)kvsel * H + h) * P + j) * HD) + pc;
    }
    reinterpret_cast<u4_t*>(kv_out + (((long)kvsel * H + h) * L + j) * HD)[pc] = *src;
  }
  if (a.last && t != T - 1) return;

  const int pos = P + t;   // keys 0 .. pos are visible
  const int j = lane & 31, half = lane >> 5;
  float dot = 0.0f;
  if (j <= pos) {
    const uint16_t* krow = j < P ? kv + ((long)h * P + j) * HD : qkv + (long)(j - P) * 3 * D + D + (long)h * HD;
    const u4_t* q4 = reinterpret_cast<const u4_t*>(qkv + (long)t * 3 * D + (long)h * HD);
    const u4_t* k4 = reinterpret_cast<const u4_t*>(krow);
    for (int pc = half * (pieces / 2); pc < (half + 1) * (pieces / 2); ++pc) {
      float qf[8], kf[8];
      widen8(q4[pc], a.dtype, qf);
      widen8(k4[pc], a.dtype, kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qf[e], kf[e], dot);
    }
  }
  // lanes j and j + 32 swap halves: both hold the key's whole dot product, in one order
  const float other = __shfl_xor(dot, 32);
  const float full = half == 0 ? dot + other : other + dot;
  const float s = j <= pos ? full * a.scale : -__builtin_inff();
  const float m = wave_max(s);
  const float e = j <= pos ? expf(s - m) : 0.0f;
  const float z = wave_sum(half == 0 ? e : 0.0f);
  const float p = e / z;

  const long row = a.last ? 0 : t;
  for (int d = lane; d < HD; d += 64) {
    float o = 0.0f;
    for (int jj = 0; jj <= pos; ++jj) {
      const float pj = __shfl(p, jj);
      const uint16_t* vrow = jj < P ? kv + (((long)H + h) * P + jj) * HD
                                    : qkv + (long)(jj - P) * 3 * D + 2 * D + (long)h * HD;
      o = fmaf(pj, bits_to_float(vrow[d], a.dtype), o);
    }
    store_elem(a.out, a.out_dtype, row * D + (long)h * HD + d, o);
  }
}

}  // namespace

hipError_t launch_attend(const AttendParams& a, hipStream_t s) {
  hipLaunchKernelGGL(attend_kernel, dim3(a.H, a.T), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlin
