// Quantized-KV decode attention for gfx950 ([p3] mlx-bun 0.0.10 -> 0.0.12,
// model/fused-decode-kernel.ts): one query position per head attends over a cache whose
// keys and values are affine-quantized along the head dimension (codes of 4 or 8 bits, one
// scale and bias per group of GS elements of a row):
//
//   s[h, n]   = sum_d q[h, d] K[c, n, d]          c = h / (H / KV)
//   out[h, d] = sum_n softmax_n(s[h, .]) V[c, n, d]
//
// The rows are split into G blocks (flash decoding).  block_kernel, one workgroup per
// (block, head): each of its 4 waves walks the block's rows four at a time (their loads
// issued together);
// lane l holds elements d = E l .. E l + E - 1 (E = D / 64, inside one group), so the
// dequantization is factored out of the dot product like the pages' qdot pattern
// (s = scale sum q code + bias sum q), the row score is an xor butterfly over the wave, and
// an online softmax keeps a running maximum, sum and value accumulator.  The waves merge in
// LDS in a fixed order into the block's unnormalized output and (max, sum).  merge_kernel
// combines the blocks in block order.  No atomics: the result is bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_internal.h"

namespace qlin {
namespace {

constexpr int kKvqThreads = 256;
constexpr int kKvqWaves = kKvqThreads / 64;
constexpr int kKvqRows = 4;   // rows a wave takes per step

__device__ __forceinline__ float half_to_float(uint16_t b, int dtype) {
  if (dtype == 1) return (float)__builtin_bit_cast(_Float16, b);
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// The E codes of lane l in row `row` (E * BITS <= 64 bits, aligned to their size).
template <int BITS, int E>
__device__ __forceinline__ void row_codes(const uint32_t* __restrict__ c, long row, int words, int lane, float out[E]) {
  constexpr uint32_t mask = (1u << BITS) - 1u;
  const long bit = (long)lane * E * BITS;
  if constexpr (E * BITS <= 32) {
    const uint32_t w = c[row * words + (bit >> 5)];
    const int sh = (int)(bit & 31);
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = (float)((w >> (sh + e * BITS)) & mask);
  } else {
    const uint32_t w0 = c[row * words + (bit >> 5)], w1 = c[row * words + (bit >> 5) + 1];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t w = e * BITS < 32 ? w0 : w1;
      out[e] = (float)((w >> ((e * BITS) & 31)) & mask);
    }
  }
}

template <int BITS, int E>
__global__ __launch_bounds__(kKvqThreads) void block_kernel(const KvqParams a) {
  constexpr int D = 64 * E;
  __shared__ float tg_max[kKvqWaves], tg_sum[kKvqWaves];
  __shared__ float tg_o[kKvqWaves * D];
  const int g = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = h / (a.H / a.KV);
  const int start = g * a.block, end = min(start + a.block, a.N);
  const int words = D * BITS / 32, groups = D / a.GS, gi = (lane * E) / a.GS;
  const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
  const uint16_t* ks = static_cast<const uint16_t*>(a.ks);
  const uint16_t* kb = static_cast<const uint16_t*>(a.kb);
  const uint16_t* vs = static_cast<const uint16_t*>(a.vs);
  const uint16_t* vb = static_cast<const uint16_t*>(a.vb);
  float qv[E], qsum = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = half_to_float(q16[(long)h * D + lane * E + e], a.q_dtype);
    qsum += qv[e];
  }
  float mx = -__builtin_inff(), sum = 0.0f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.0f;
  // wave wv takes rows start + U wv + 4 U j + u (u < U): the U rows' loads are all issued
  // before their scores are reduced, and their online-softmax update is one step
  for (int n0 = start + kKvqRows * wv; n0 < end; n0 += kKvqWaves * kKvqRows) {
    float kcode[kKvqRows][E], vcode[kKvqRows][E], ksc[kKvqRows], kbi[kKvqRows], vsc[kKvqRows], vbi[kKvqRows];
#pragma unroll
    for (int u = 0; u < kKvqRows; ++u) {
      const long row = (long)c * a.N + min(n0 + u, end - 1);   // rows past the block: masked below
      row_codes<BITS, E>(a.kc, row, words, lane, kcode[u]);
      row_codes<BITS, E>(a.vc, row, words, lane, vcode[u]);
      ksc[u] = half_to_float(ks[row * groups + gi], a.sb_dtype);
      kbi[u] = half_to_float(kb[row * groups + gi], a.sb_dtype);
      vsc[u] = half_to_float(vs[row * groups + gi], a.sb_dtype);
      vbi[u] = half_to_float(vb[row * groups + gi], a.sb_dtype);
    }
    float s[kKvqRows];
#pragma unroll
    for (int u = 0; u < kKvqRows; ++u) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) dot = fmaf(qv[e], kcode[u][e], dot);
      s[u] = wave_sum64(fmaf(ksc[u], dot, kbi[u] * qsum));
    }
    float m = mx;
#pragma unroll
    for (int u = 0; u < kKvqRows; ++u)
      if (n0 + u < end) m = fmaxf(m, s[u]);
    const float f = expf(mx - m);
    float p[kKvqRows];
#pragma unroll
    for (int u = 0; u < kKvqRows; ++u) p[u] = n0 + u < end ? expf(s[u] - m) : 0.0f;
    float ps = sum * f;
#pragma unroll
    for (int u = 0; u < kKvqRows; ++u) ps += p[u];
    sum = ps;
    mx = m;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float acc = o[e] * f;
#pragma unroll
      for (int u = 0; u < kKvqRows; ++u) acc = fmaf(p[u], fmaf(vcode[u][e], vsc[u], vbi[u]), acc);
      o[e] = acc;
    }
  }
  if (lane == 0) {
    tg_max[wv] = mx;
    tg_sum[wv] = sum;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) tg_o[wv * D + lane * E + e] = o[e];
  __syncthreads();
  if (wv == 0) {
    float M = tg_max[0];
    for (int w = 1; w < kKvqWaves; ++w) M = fmaxf(M, tg_max[w]);
    float wgt[kKvqWaves], S = 0.0f;
    for (int w = 0; w < kKvqWaves; ++w) {
      wgt[w] = tg_max[w] == -__builtin_inff() ? 0.0f : expf(tg_max[w] - M);   // a wave without rows
      S = fmaf(tg_sum[w], wgt[w], S);
    }
    const long base = ((long)h * a.G + g) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = lane * E + e;
      float v = 0.0f;
      for (int w = 0; w < kKvqWaves; ++w) v = fmaf(tg_o[w * D + d], wgt[w], v);
      a.opart[base + d] = v;
    }
    if (lane == 0) {
      a.stats[((long)h * a.G + g) * 2 + 0] = M;
      a.stats[((long)h * a.G + g) * 2 + 1] = S;
    }
  }
}

// out[h, d] = sum_g opart[h, g, d] e^(M_g - M) / sum_g S_g e^(M_g - M), blocks in order.
__global__ __launch_bounds__(512) void merge_kernel(const KvqParams a) {
  const int h = blockIdx.x, d = threadIdx.x, D = a.D;
  if (d >= D) return;
  const float* st = a.stats + (long)h * a.G * 2;
  float M = st[0];
  for (int g = 1; g < a.G; ++g) M = fmaxf(M, st[2 * g]);
  float den = 0.0f, o = 0.0f;
  for (int g = 0; g < a.G; ++g) {
    const float w = expf(st[2 * g] - M);
    den = fmaf(st[2 * g + 1], w, den);
    o = fmaf(a.opart[((long)h * a.G + g) * D + d], w, o);
  }
  const float v = o / den;
  const long idx = (long)h * D + d;
  if (a.out_dtype == 0) static_cast<float*>(a.out)[idx] = v;
  else if (a.out_dtype == 1) static_cast<_Float16*>(a.out)[idx] = (_Float16)v;
  else static_cast<__bf16*>(a.out)[idx] = (__bf16)v;
}

template <int BITS>
hipError_t launch_block(const KvqParams& a, hipStream_t s) {
  const dim3 grid(a.G, a.H);
  switch (a.D) {
    case 64: hipLaunchKernelGGL((block_kernel<BITS, 1>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((block_kernel<BITS, 2>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL((block_kernel<BITS, 4>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 512: hipLaunchKernelGGL((block_kernel<BITS, 8>), grid, dim3(kKvqThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kvq_decode(const KvqParams& a, hipStream_t s) {
  const hipError_t e = a.bits == 4 ? launch_block<4>(a, s) : launch_block<8>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.H), dim3(a.D), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlin
