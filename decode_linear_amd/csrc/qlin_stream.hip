// Streaming-read ceiling of the device: a plain read of a buffer with 16-byte loads, the
// access the weight stream of the fused linear makes, with no arithmetic beyond an XOR
// fold that keeps the loads alive.  Its time over the same number of bytes is the HBM
// rate this device reaches for a pure read, next to which the fused kernel's rate reads.
#include "qlin_internal.h"

namespace qlin {

namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
constexpr int kReadThreads = 512;

__device__ __forceinline__ uint32_t fold(const u4_t v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Block b XOR-folds the 16-byte words b*512 + t + k*stride (stride = grid*512), U loads in
// flight per thread and round (non-temporal loads when NT), and writes the fold of the whole
// block to partial[b].  Words are read once each.
template <int U, bool NT>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u4_t* __restrict__ a, int64_t words,
                                                                   uint32_t* __restrict__ partial) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (U - 1) * stride < words; i += U * stride) {
    u4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(a + i + u * stride) : a[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
  }
  for (; i < words; i += stride) acc ^= fold(a[i]);
  // the block's fold: within the wave by lane exchanges, across the 8 waves through LDS
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  __shared__ uint32_t wf[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) wf[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t f = 0u;
#pragma unroll
    for (int w = 0; w < kReadThreads / 64; ++w) f ^= wf[w];
    partial[blockIdx.x] = f;
  }
}

template <int U>
hipError_t launch_u(const void* buf, int64_t bytes, uint32_t* partial, int grid, bool nt, hipStream_t s) {
  if (nt)
    hipLaunchKernelGGL((stream_read_kernel<U, true>), dim3(grid), dim3(kReadThreads), 0, s,
                       reinterpret_cast<const u4_t*>(buf), bytes / 16, partial);
  else
    hipLaunchKernelGGL((stream_read_kernel<U, false>), dim3(grid), dim3(kReadThreads), 0, s,
                       reinterpret_cast<const u4_t*>(buf), bytes / 16, partial);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* partial, int grid, int unroll, bool nt,
                              hipStream_t s) {
  switch (unroll) {
    case 1: return launch_u<1>(buf, bytes, partial, grid, nt, s);
    case 2: return launch_u<2>(buf, bytes, partial, grid, nt, s);
    case 4: return launch_u<4>(buf, bytes, partial, grid, nt, s);
    case 8: return launch_u<8>(buf, bytes, partial, grid, nt, s);
    case 16: return launch_u<16>(buf, bytes, partial, grid, nt, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlin
