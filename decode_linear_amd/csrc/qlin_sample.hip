// sample for gfx950: one sampling step of the depth decoder ([p1] maya-mac
// src/maya_mac/mlx_kernels.py, `_SAMPLE` and `sample()`).
//
//   key(f)  = order-preserving 32-bit key of the fp32 logit f (bits u; ~u when negative,
//             u | 2^31 otherwise), so larger logits have larger keys and -0 < +0
//   kth     = the top_k-th largest key, found exactly by a radix select (4 passes of 8 bits)
//   code    = argmax over the codes with key >= kth (ties with the k-th all kept) of
//             fl32(fl32(f * inv_temp) + gumbel), the smaller index on equal scores; a NaN
//             score never wins, and no number among the kept scores gives -1
//   out     = the prefix rows, then (with a table) the table row of the code (zeros for -1)
//
// Mapping: one workgroup of 256 threads (4 waves); thread t holds the keys of codes
// t, t + 256, ... in registers (n <= 8192).  A radix pass counts digits of the keys that
// still match the selected prefix into a 256-bin LDS histogram (integer LDS atomics: the
// counts do not depend on their order), and wave 0 scans the bins from the top with a lane
// prefix sum to find the digit that holds the need-th largest key.  The argmax is a
// per-thread scan, an xor butterfly over each wave (a total order on (score, index)) and a
// fixed-order pass over the four waves.  The rows are copied with 16-byte accesses, the
// prefix first of all (it does not depend on the code).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_internal.h"

namespace qlin {
namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
constexpr int kSampleThreads = 256;
constexpr int kSamplePerThread = kSampleMaxCodes / kSampleThreads;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ float logit_at(const SampleParams& a, int i) {
  if (a.logit_dtype == 0) return static_cast<const float*>(a.logits)[i];
  const uint16_t b = static_cast<const uint16_t*>(a.logits)[i];
  if (a.logit_dtype == 1) return (float)__builtin_bit_cast(_Float16, b);
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// (s, i) beats (bs, bi): a larger score, or an equal score at a smaller index.  Scores are
// never NaN on the winning side (a NaN compares false both ways and is never taken).
__device__ __forceinline__ bool beats(float s, uint32_t i, float bs, uint32_t bi) {
  return s > bs || (s == bs && i < bi);
}

__global__ __launch_bounds__(kSampleThreads) void sample_kernel(const SampleParams a) {
#pragma clang fp contract(off)
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_need;
  __shared__ float best_s[kSampleThreads / 64];
  __shared__ uint32_t best_i[kSampleThreads / 64];
  __shared__ int32_t sh_code;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = a.n;
  // the prefix rows do not depend on the code: they are copied first, their loads in
  // flight together, while the keys load and the selection runs
  const long W = (long)a.D * a.es / 16;   // 16-byte pieces per row
  u4_t* out = static_cast<u4_t*>(a.out);
  if (a.copy_prefix) {
    const u4_t* pre = static_cast<const u4_t*>(a.prefix);
    const long total = (long)a.n_prev * W;
    long v = tid;
    for (; v + 7 * kSampleThreads < total; v += 8 * kSampleThreads) {
      u4_t t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = pre[v + u * kSampleThreads];
#pragma unroll
      for (int u = 0; u < 8; ++u) out[v + u * kSampleThreads] = t[u];
    }
    for (; v < total; v += kSampleThreads) out[v] = pre[v];
  }

  uint32_t key[kSamplePerThread];
#pragma unroll
  for (int e = 0; e < kSamplePerThread; ++e) {
    const int i = tid + kSampleThreads * e;
    key[e] = i < n ? order_key(logit_at(a, i)) : 0u;
  }
  if (tid == 0) {
    sh_prefix = 0u;
    sh_need = (uint32_t)a.top_k;
  }
  // radix select of the top_k-th largest key, 8 bits per pass from the top
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0u;   // 256 threads, 256 bins
    __syncthreads();  // also publishes sh_prefix / sh_need of the previous pass
    const uint32_t prefix = sh_prefix;
#pragma unroll
    for (int e = 0; e < kSamplePerThread; ++e) {
      const int i = tid + kSampleThreads * e;
      const bool match = pass == 0 ? true : (key[e] >> (shift + 8)) == prefix;
      if (i < n && match) atomicAdd(&hist[(key[e] >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    if (wv == 0) {
      // lane l holds bins 255 - 4l .. 252 - 4l, in descending order
      uint32_t c[4], tot = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - (4 * lane + j)];
        tot += c[j];
      }
      uint32_t incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += t;
      }
      const uint32_t before = incl - tot, need = sh_need;
      if (before < need && need <= before + tot) {   // exactly one lane: need <= the candidates
        uint32_t run = before;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (need <= run + c[j]) {
            sh_prefix = (prefix << 8) | (uint32_t)(255 - (4 * lane + j));
            sh_need = need - run;
            break;
          }
          run += c[j];
        }
      }
    }
    __syncthreads();
  }
  const uint32_t kth = sh_prefix;
  // Gumbel-max over the kept codes
  float bs = -__builtin_inff();
  uint32_t bi = 0xFFFFFFFFu;
#pragma unroll
  for (int e = 0; e < kSamplePerThread; ++e) {
    const int i = tid + kSampleThreads * e;
    if (i < n && key[e] >= kth) {
      const float scaled = key_value(key[e]) * a.inv_temp;   // one fp32 rounding
      const float s = scaled + a.gumbel[i];                  // and another (no contraction)
      if (beats(s, (uint32_t)i, bs, bi)) {
        bs = s;
        bi = (uint32_t)i;
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float os = __shfl_xor(bs, m, 64);
    const uint32_t oi = (uint32_t)__shfl_xor((int)bi, m, 64);
    if (beats(os, oi, bs, bi)) {
      bs = os;
      bi = oi;
    }
  }
  if (lane == 0) {
    best_s[wv] = bs;
    best_i[wv] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    float s = best_s[0];
    uint32_t i = best_i[0];
    for (int w = 1; w < kSampleThreads / 64; ++w)
      if (beats(best_s[w], best_i[w], s, i)) {
        s = best_s[w];
        i = best_i[w];
      }
    const int32_t c = i == 0xFFFFFFFFu ? -1 : (int32_t)i;
    sh_code = c;
    *a.code = c;
  }
  __syncthreads();
  // the code's table row after the prefix
  if (a.table) {
    const int32_t c = sh_code;
    const u4_t* row = static_cast<const u4_t*>(a.table) + (long)(c < 0 ? 0 : c) * W;
    for (long v = tid; v < W; v += kSampleThreads)
      out[(long)a.n_prev * W + v] = c < 0 ? (u4_t){0u, 0u, 0u, 0u} : row[v];
  }
}

}  // namespace

hipError_t launch_sample(const SampleParams& a, hipStream_t s) {
  hipLaunchKernelGGL(sample_kernel, dim3(1), dim3(kSampleThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlin
