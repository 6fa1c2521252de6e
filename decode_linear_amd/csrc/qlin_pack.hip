// Affine group quantizer (pack) and dequantizer (unpack) kernels.
//
// Format ([p1] maya-mac src/maya_mac/mlx_kernels.py, the 8-bit load of `_linear_kernel`;
// [p3] mlx-bun 0.0.10 -> 0.0.12, model/fused-decode-kernel.ts for 4 bits): codes packed
// low bits first, 32/bits per uint32 word, one fp16 scale and bias per group of 64 k.
// The quantizer itself is not printed on the pages; the library fixes it as
//   s = fp16(fl32(fl32(hi - lo) / (2^bits - 1))),  b = fp16(lo),
//   q = s == 0 ? 0 : clamp(rint(fl32(fl32(w - b) / s)), 0, 2^bits - 1)
// with IEEE binary32 steps (correctly rounded division, no contraction) and ties to even.
#include "qlin_internal.h"

namespace qlin {

namespace {

#pragma clang fp contract(off)

__global__ void pack_kernel(const float* __restrict__ w, int64_t N, int64_t K, int bits,
                            uint32_t* __restrict__ codes, uint16_t* __restrict__ scales,
                            uint16_t* __restrict__ biases, int32_t* flag) {
  const int64_t G = K / 64;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= N * G) return;
  const int64_t n = gid / G, g = gid - n * G;
  const float* v = w + n * K + g * 64;
  float lo = v[0], hi = v[0];
  bool finite = true;
  for (int j = 0; j < 64; ++j) {
    const float a = v[j];
    finite = finite && __builtin_isfinite(a);
    lo = a < lo ? a : lo;
    hi = a > hi ? a : hi;
  }
  const int per = 32 / bits;
  const int64_t words_per_row = K / per;
  uint32_t* out = codes + n * words_per_row + g * (64 / per);
  const float qmax = (float)((1 << bits) - 1);
  bool bad = !finite;
  _Float16 s16 = (_Float16)0.0f, b16 = (_Float16)0.0f;
  if (!bad) {
    const float range = hi - lo;
    const float s32 = range / qmax;
    s16 = (_Float16)s32;
    b16 = (_Float16)lo;
    bad = !__builtin_isfinite((float)s16) || !__builtin_isfinite((float)b16);
  }
  if (bad) {
    for (int i = 0; i < 64 / per; ++i) out[i] = 0u;
    scales[n * G + g] = 0x0000;
    biases[n * G + g] = 0x7E00;
    if (flag) *flag = 1;
    return;
  }
  scales[n * G + g] = __builtin_bit_cast(uint16_t, s16);
  biases[n * G + g] = __builtin_bit_cast(uint16_t, b16);
  const float s = (float)s16, b = (float)b16;
  for (int i = 0; i < 64 / per; ++i) {
    uint32_t word = 0u;
    for (int j = 0; j < per; ++j) {
      uint32_t q = 0u;
      if (s != 0.0f) {
        const float diff = v[i * per + j] - b;
        const float ratio = diff / s;
        float r = __builtin_rintf(ratio);
        r = r < 0.0f ? 0.0f : (r > qmax ? qmax : r);
        q = (uint32_t)r;
      }
      word |= q << (bits * j);
    }
    out[i] = word;
  }
}

__global__ void unpack_kernel(const void* __restrict__ data, const uint16_t* __restrict__ scales,
                              const uint16_t* __restrict__ biases, int bits, int dtype, int64_t N, int64_t K,
                              float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * K) return;
  const int64_t n = i / K, k = i - n * K;
  if (bits == 16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(data)[i];
    out[i] = dtype == 1 ? (float)__builtin_bit_cast(_Float16, h) : __builtin_bit_cast(float, (uint32_t)h << 16);
    return;
  }
  const int per = 32 / bits;
  const uint32_t word = reinterpret_cast<const uint32_t*>(data)[n * (K / per) + k / per];
  const uint32_t q = (word >> (bits * (k % per))) & ((1u << bits) - 1u);
  const int64_t gi = n * (K / 64) + k / 64;
  const float s = (float)__builtin_bit_cast(_Float16, scales[gi]);
  const float b = (float)__builtin_bit_cast(_Float16, biases[gi]);
  out[i] = __builtin_fmaf((float)q, s, b);
}

}  // namespace

hipError_t launch_pack(const float* w, int64_t N, int64_t K, int bits, uint32_t* codes, uint16_t* scales,
                       uint16_t* biases, int32_t* flag, hipStream_t s) {
  const int64_t groups = N * (K / 64);
  const int threads = 256;
  const int64_t blocks = (groups + threads - 1) / threads;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, w, N, K, bits, codes, scales, biases, flag);
  return hipGetLastError();
}

hipError_t launch_unpack(const void* data, const uint16_t* scales, const uint16_t* biases, int bits, int dtype,
                         int64_t N, int64_t K, float* out, hipStream_t s) {
  const int64_t total = N * K;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, data, scales, biases, bits, dtype, N, K, out);
  return hipGetLastError();
}

}  // namespace qlin
