// Quantized-KV decode attention for gfx950 ([p3] mlx-bun 0.0.10 -> 0.0.12,
// model/fused-decode-kernel.ts): one query position per head attends over a cache whose
// keys and values are affine-quantized along the head dimension (codes of 4 or 8 bits, one
// scale and bias per group of GS elements of a row):
//
//   s[h, n]   = sum_d q[h, d] K[c, n, d]          c = h / (H / KV)
//   out[h, d] = sum_n softmax_n(s[h, .]) V[c, n, d]
//
// The rows are split into G blocks (flash decoding).  block_kernel, one workgroup per
// (block, head): a wave takes 64 / L rows per step, L = (bytes of a row of codes) / 16
// lanes per row, each lane one 16-byte slice (32 4-bit or 16 8-bit codes, inside one
// quantization group), so the dequantization factors out of the dot product like the
// pages' qdot pattern (s = scale sum q code + bias sum q); the row's score is an xor
// butterfly over its L lanes, and an online softmax over the step's rows keeps a running
// maximum, weight sum and per-slice value accumulator, summed over the row slots at the
// end of the block.  The waves merge in
// LDS in a fixed order into the block's unnormalized output and (max, sum).  merge_kernel
// combines the blocks in block order.  No atomics: the result is bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "qlin.h"
#include "qlin_internal.h"

namespace qlin {
namespace {

constexpr int kKvqThreads = 256;
constexpr int kKvqWaves = kKvqThreads / 64;
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_to_float(uint16_t b, int dtype) {
  if (dtype == 1) return (float)__builtin_bit_cast(_Float16, b);
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int BITS, int D>
__global__ __launch_bounds__(kKvqThreads) void block_kernel(const KvqParams a) {
  constexpr int RB = D * BITS / 8;      // bytes of a row of codes
  constexpr int LPR = RB / 16;          // lanes per row: each takes 16 bytes
  constexpr int R = 64 / LPR;           // rows a wave takes per step
  constexpr int EL = 128 / BITS;        // elements per lane (inside one quantization group)
  constexpr int E = D / 64;             // elements per lane in the merge
  constexpr uint32_t mask = (1u << BITS) - 1u;
  static_assert(LPR >= 2 && LPR <= 32 && EL * LPR == D, "16-byte lane slices");
  __shared__ float tg_max[kKvqWaves], tg_sum[kKvqWaves];
  __shared__ float tg_o[kKvqWaves * D];
  const int g = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / LPR, j = lane % LPR;   // row slot, slice of the row
  const int c = h / (a.H / a.KV);
  const int start = g * a.block, end = min(start + a.block, a.N);
  const int groups = D / a.GS, gi = (j * EL) / a.GS;
  const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
  const uint16_t* ks = static_cast<const uint16_t*>(a.ks);
  const uint16_t* kb = static_cast<const uint16_t*>(a.kb);
  const uint16_t* vs = static_cast<const uint16_t*>(a.vs);
  const uint16_t* vb = static_cast<const uint16_t*>(a.vb);
  const u4_t* kc = reinterpret_cast<const u4_t*>(a.kc);
  const u4_t* vc = reinterpret_cast<const u4_t*>(a.vc);
  float qv[EL], qsum = 0.0f;
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    qv[e] = half_to_float(q16[(long)h * D + j * EL + e], a.q_dtype);
    qsum += qv[e];
  }
  float mx = -__builtin_inff(), lsum = 0.0f, o[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) o[e] = 0.0f;
  for (int n0 = start + R * wv; n0 < end; n0 += kKvqWaves * R) {
    const int n = n0 + slot;
    const bool live = n < end;
    const long row = (long)c * a.N + (live ? n : end - 1);   // rows past the block: masked below
    const u4_t kw = kc[row * LPR + j], vw = vc[row * LPR + j];
    const float ksc = half_to_float(ks[row * groups + gi], a.sb_dtype), kbi = half_to_float(kb[row * groups + gi], a.sb_dtype);
    const float vsc = half_to_float(vs[row * groups + gi], a.sb_dtype), vbi = half_to_float(vb[row * groups + gi], a.sb_dtype);
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < EL; ++e) dot = fmaf(qv[e], (float)((kw[(e * BITS) >> 5] >> ((e * BITS) & 31)) & mask), dot);
    float s = fmaf(ksc, dot, kbi * qsum);
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m, 64);   // the row's score on its LPR lanes
    float smax = live ? s : -__builtin_inff();
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) smax = fmaxf(smax, __shfl_xor(smax, m, 64));   // over the step's rows
    const float mnew = fmaxf(mx, smax);
    const float f = expf(mx - mnew), p = live ? expf(s - mnew) : 0.0f;
    lsum = fmaf(lsum, f, j == 0 ? p : 0.0f);   // one lane per row carries its weight
    mx = mnew;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const float v = fmaf((float)((vw[(e * BITS) >> 5] >> ((e * BITS) & 31)) & mask), vsc, vbi);
      o[e] = fmaf(o[e], f, p * v);
    }
  }
  // sum over the row slots: lanes of one slice, then the wave's weight sum
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < EL; ++e) o[e] += __shfl_xor(o[e], m, 64);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) lsum += __shfl_xor(lsum, m, 64);
  if (lane == 0) {
    tg_max[wv] = mx;
    tg_sum[wv] = lsum;
  }
  if (slot == 0) {
#pragma unroll
    for (int e = 0; e < EL; ++e) tg_o[wv * D + j * EL + e] = o[e];
  }
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

// A workgroup-wide reduction of one value per thread in a fixed order: an xor butterfly in
// each wave, then the four waves' results in wave order, read by every thread.
template <bool MAX>
__device__ __forceinline__ float merge_reduce(float v, float* part) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(v, m, 64);
    v = MAX ? fmaxf(v, o) : v + o;
  }
  __syncthreads();   // earlier readers of part are done
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = part[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = MAX ? fmaxf(r, part[w]) : r + part[w];
  return r;
}

// out[h, d] = sum_g opart[h, g, d] e^(M_g - M) / sum_g S_g e^(M_g - M), one workgroup per
// head.  M and the denominator are fixed-order reductions (thread t takes blocks t, t + 256,
// ... in order, then merge_reduce: a butterfly per wave and the waves in order; one thread
// walking 256 LDS partials cost about 2.5 us); the block weights e^(M_g - M) go to LDS in
// chunks, and each thread sums its columns over the blocks in block order with the loads of
// a chunk independent of each other.
constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 4096;
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const KvqParams a) {
  __shared__ float part[kMergeThreads];
  __shared__ float wgt[kMergeChunk];
  const int h = blockIdx.x, t = threadIdx.x, D = a.D, G = a.G;
  const float* st = a.stats + (long)h * G * 2;
  // up to 256 blocks (every head with at most 32768 rows): each thread reads its block's
  // statistics once and keeps them for the weights
  const bool one = G <= kMergeThreads;
  float m_t = -__builtin_inff(), s_t = 0.0f;
  if (one && t < G) {
    m_t = st[2 * t];
    s_t = st[2 * t + 1];
  }
  float m = m_t;
  if (!one)
    for (int g = t; g < G; g += kMergeThreads) m = fmaxf(m, st[2 * g]);
  const float M = merge_reduce<true>(m, part);
  const float w_t = expf(m_t - M);
  float den = one ? fmaf(s_t, w_t, 0.0f) : 0.0f;
  if (!one)
    for (int g = t; g < G; g += kMergeThreads) den = fmaf(st[2 * g + 1], expf(st[2 * g] - M), den);
  const float den_all = merge_reduce<false>(den, part);
  float o0 = 0.0f, o1 = 0.0f;   // columns t and t + 256 (D <= 512)
  const float* op = a.opart + (long)h * G * D;
  for (int g0 = 0; g0 < G; g0 += kMergeChunk) {
    const int gn = min(kMergeChunk, G - g0);
    __syncthreads();   // the previous chunk's weights are read
    if (one) {
      if (t < G) wgt[t] = w_t;
    } else {
      for (int i = t; i < gn; i += kMergeThreads) wgt[i] = expf(st[2 * (g0 + i)] - M);
    }
    __syncthreads();
    if (t < D) {
#pragma unroll 16
      for (int i = 0; i < gn; ++i) o0 = fmaf(op[(long)(g0 + i) * D + t], wgt[i], o0);
    }
    if (t + kMergeThreads < D) {
#pragma unroll 16
      for (int i = 0; i < gn; ++i) o1 = fmaf(op[(long)(g0 + i) * D + t + kMergeThreads], wgt[i], o1);
    }
  }
  for (int k = 0; k < 2; ++k) {
    const int d = t + k * kMergeThreads;
    if (d >= D) continue;
    const float v = (k == 0 ? o0 : o1) / den_all;
    const long idx = (long)h * D + d;
    if (a.out_dtype == 0) static_cast<float*>(a.out)[idx] = v;
    else if (a.out_dtype == 1) static_cast<_Float16*>(a.out)[idx] = (_Float16)v;
    else static_cast<__bf16*>(a.out)[idx] = (__bf16)v;
  }
}

template <int BITS>
hipError_t launch_block(const KvqParams& a, hipStream_t s) {
  const dim3 grid(a.G, a.H);
  switch (a.D) {
    case 64: hipLaunchKernelGGL((block_kernel<BITS, 64>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((block_kernel<BITS, 128>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL((block_kernel<BITS, 256>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 512: hipLaunchKernelGGL((block_kernel<BITS, 512>), grid, dim3(kKvqThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// The partials of qlin_kvq_decode_noalloc: one copy of this array lives on every GPU the
// library runs on.  Host code never passes its name to a kernel (on the host the name is a
// stand-in, not a device address): it passes the address kvq_scratch looked up.
static __device__ __align__(256) float scratch[QLIN_KVQ_SCRATCH_BYTES / sizeof(float)];

hipError_t kvq_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_kvq_decode(const KvqParams& a, hipStream_t s) {
  const hipError_t e = a.bits == 4 ? launch_block<4>(a, s) : launch_block<8>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.H), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlin
