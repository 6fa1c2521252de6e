// Quantized-KV decode attention for gfx950 ([p3] mlx-bun 0.0.10 -> 0.0.12,
// model/fused-decode-kernel.ts): one query position per head attends over a cache whose
// keys and values are affine-quantized along the head dimension (codes of 4 or 8 bits, one
// scale and bias per group of GS elements of a row):
//
//   s[h, n]   = sum_d q[h, d] K[c, n, d]          c = h / (H / KV)
//   out[h, d] = sum_n softmax_n(s[h, .]) V[c, n, d]
//
// The rows are split into G blocks (flash decoding).  block_kernel takes one workgroup per
// (block, KV head, pair of the query heads that share it), so each cache row is read once
// for both heads (a head count that does not pair up takes one head per workgroup).  A wave
// takes 64 / L rows per step, L = (bytes of a row of codes) / 16 lanes per row, each lane
// one 16-byte slice (32 4-bit or 16 8-bit codes, inside one quantization group), so the
// dequantization factors out of the dot product like the pages' qdot pattern (s = scale
// sum q code + bias sum q); the row's score is an xor butterfly over its L lanes, and an
// online softmax per head over the step's rows keeps a running maximum, weight sum and
// per-slice value accumulator (each value decoded once for both heads), summed over the
// row slots at the end of the block.  The waves merge in LDS in a fixed order into the
// block's unnormalized output and (max, sum) per head.  merge_kernel combines the blocks in
// a fixed order (four quarters of the block range, each in block order, then the quarters in
// order).  No atomics: the result is bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "qlin.h"
#include "qlin_internal.h"

namespace qlin {
namespace {

// Eight waves per workgroup over 256-row blocks (two waves per SIMD, 32 rows per wave in two
// rounds): 13.58-13.64 -> 13.45-13.52 us against four waves over 128 rows, the merge taking
// half as many blocks.
constexpr int kKvqThreads = 512;
constexpr int kKvqWaves = kKvqThreads / 64;
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_to_float(uint16_t b, int dtype) {
  if (dtype == 1) return (float)__builtin_bit_cast(_Float16, b);
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// Cross-lane combines without LDS: v op v[lane ^ 2^B], the same value on both lanes of each
// pair.  Bits 0 and 1 are DPP quad permutes, bit 2 two row shifts and a select, bit 3 a row
// rotation by 8, bits 4 and 5 the gfx950 row swaps (v_permlane16_swap pairs rows 0-1 and
// 2-3, v_permlane32_swap the two halves; each returns both rows of a pair, so op over the two
// results combines the pair).
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int B, bool MAX> __device__ __forceinline__ float xcomb(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (B == 0) return op(v, dpp_f<0xB1>(v));                 // quad_perm [1, 0, 3, 2]
  else if constexpr (B == 1) return op(v, dpp_f<0x4E>(v));            // quad_perm [2, 3, 0, 1]
  else if constexpr (B == 2) {
    const float dn = dpp_f<0x114>(v), up = dpp_f<0x104>(v);           // row_shr:4, row_shl:4
    return op(v, (threadIdx.x & 4) ? dn : up);
  } else if constexpr (B == 3) return op(v, dpp_f<0x128>(v));         // row_ror:8
  else if constexpr (B == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    return op(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
    return op(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
  }
}
// op over the lanes that differ from this one only in bits [LO, HI) of the lane index, in a
// fixed order (bit LO first); every such lane ends with the same value.
template <int LO, int HI, bool MAX> __device__ __forceinline__ float lane_reduce(float v) {
  if constexpr (LO < HI) return lane_reduce<LO + 1, HI, MAX>(xcomb<LO, MAX>(v));
  else return v;
}
constexpr int log2i(int v) { return v <= 1 ? 0 : 1 + log2i(v / 2); }

// The four bytes of w as floats, f[0], f[stride], f[2 stride], f[3 stride] (v_cvt_f32_ubyteN
// converts byte N directly; the compiler otherwise extracts a narrower field first).
__device__ __forceinline__ void bytes_to_float(uint32_t w, float* f, int stride) {
  float b0, b1, b2, b3;
  asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(b0) : "v"(w));
  asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(b1) : "v"(w));
  asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(b2) : "v"(w));
  asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(b3) : "v"(w));
  f[0] = b0;
  f[stride] = b1;
  f[2 * stride] = b2;
  f[3 * stride] = b3;
}

// One level of a reduce-scatter over lane bit B: u holds N values; afterwards the first N / 2
// hold the sums (this lane + the lane across bit B) of elements [0, N/2) on lanes whose bit B
// is 0 and of elements [N/2, N) on lanes whose bit B is 1.  Bits 4 and 5 use the row swaps,
// which hand each lane exactly the pair it needs; bits 0-3 select the half the partner keeps
// and fetch the partner's selection with a DPP move.
template <int B, int N> __device__ __forceinline__ void scatter_level(float* u) {
  constexpr int H = N / 2;
  if constexpr (B >= 4) {
#pragma unroll
    for (int e = 0; e < H; ++e) {
      const int lo = __builtin_bit_cast(int, u[e]), hi = __builtin_bit_cast(int, u[e + H]);
      const auto r = B == 5 ? __builtin_amdgcn_permlane32_swap(lo, hi, false, false)
                            : __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
      u[e] = __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
    }
  } else {
    const bool up = (threadIdx.x >> B) & 1;
#pragma unroll
    for (int e = 0; e < H; ++e) {
      const float keep = up ? u[e + H] : u[e], give = up ? u[e] : u[e + H];
      float other;
      if constexpr (B == 0) other = dpp_f<0xB1>(give);
      else if constexpr (B == 1) other = dpp_f<0x4E>(give);
      else if constexpr (B == 2) {
        const float dn = dpp_f<0x114>(give), upv = dpp_f<0x104>(give);
        other = up ? dn : upv;
      } else other = dpp_f<0x128>(give);
      u[e] = keep + other;
    }
  }
}
// Reduce-scatter of N values over lane bits [LO, 6), highest bit first: the lane keeps
// N >> (6 - LO) sums; its k-th is element k + scatter_base<LO>(lane) of the original N.
template <int LO, int N> __device__ __forceinline__ void reduce_scatter(float* u) {
  if constexpr (LO < 6) {
    if constexpr (6 - 1 >= LO) scatter_level<5, N>(u);
    if constexpr (LO <= 4) scatter_level<4, N / 2>(u);
    if constexpr (LO <= 3) scatter_level<3, N / 4>(u);
    if constexpr (LO <= 2) scatter_level<2, N / 8>(u);
    if constexpr (LO <= 1) scatter_level<1, N / 16>(u);
    if constexpr (LO <= 0) scatter_level<0, N / 32>(u);
  }
}
template <int LO, int N> __device__ __forceinline__ int scatter_base(int lane) {
  int base = 0, n = N;
#pragma unroll
  for (int b = 5; b >= LO; --b) {
    n /= 2;
    if ((lane >> b) & 1) base += n;
  }
  return base;
}

// One workgroup per (block g, KV head c, chunk z of QC query heads sharing c): the block's
// rows of c are read once for all QC heads (each key slice's dot product is taken against
// every head's query, and each value is decoded once and added to every head's accumulator).
template <int BITS, int D, int QC, int SBT, int QT>
__global__ __launch_bounds__(kKvqThreads) void block_kernel(const KvqParams a) {
  constexpr int P = 2;                  // steps whose rows are in flight at once
  constexpr int RB = D * BITS / 8;      // bytes of a row of codes
  constexpr int LPR = RB / 16;          // lanes per row: each takes 16 bytes
  constexpr int LB = log2i(LPR);        // lane-index bits of the slice (the rest: the row slot)
  constexpr int R = 64 / LPR;           // rows a wave takes per step
  constexpr int EL = 128 / BITS;        // elements per lane (inside one quantization group)
  constexpr int E = D / 64;             // elements per lane in the merge
  constexpr uint32_t mask = (1u << BITS) - 1u;
  static_assert(LPR >= 2 && LPR <= 32 && EL * LPR == D && (1 << LB) == LPR, "16-byte lane slices");
  __shared__ float tg_max[QC][kKvqWaves], tg_sum[QC][kKvqWaves];
  __shared__ float tg_o[QC][kKvqWaves * D];
  const int g = blockIdx.x, c = blockIdx.y;
  const int h0 = c * (a.H / a.KV) + (int)blockIdx.z * QC;   // first query head of this workgroup
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / LPR, j = lane % LPR;   // row slot, slice of the row
  const int start = g * a.block, end = min(start + a.block, a.N);
  const int groups = D / a.GS, gi = (j * EL) / a.GS;
  const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
  // the block's rows of KV head c: bases shared by the workgroup, 32-bit offsets per lane
  const long rbase = (long)c * a.N + start;
  const uint16_t* ks = static_cast<const uint16_t*>(a.ks) + rbase * groups;
  const uint16_t* kb = static_cast<const uint16_t*>(a.kb) + rbase * groups;
  const uint16_t* vs = static_cast<const uint16_t*>(a.vs) + rbase * groups;
  const uint16_t* vb = static_cast<const uint16_t*>(a.vb) + rbase * groups;
  const u4_t* kc = reinterpret_cast<const u4_t*>(a.kc) + rbase * LPR;
  const u4_t* vc = reinterpret_cast<const u4_t*>(a.vc) + rbase * LPR;
  const int nloc = end - start;   // rows of the block (>= 1)
  // this lane's EL query elements of each head: 16-byte loads when q is 16-byte aligned
  float qv[QC][EL], qsum[QC];
  if (a.q_vec) {
#pragma unroll
    for (int i = 0; i < QC; ++i)
#pragma unroll
      for (int u = 0; u < EL / 8; ++u) {
        const u4_t w = reinterpret_cast<const u4_t*>(q16 + (long)(h0 + i) * D + j * EL)[u];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[i][8 * u + e] = half_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, QT);
      }
  } else {
#pragma unroll
    for (int i = 0; i < QC; ++i)
#pragma unroll
      for (int e = 0; e < EL; ++e) qv[i][e] = half_to_float(q16[(long)(h0 + i) * D + j * EL + e], QT);
  }
#pragma unroll
  for (int i = 0; i < QC; ++i) {
    qsum[i] = 0.0f;
#pragma unroll
    for (int e = 0; e < EL; ++e) qsum[i] += qv[i][e];
  }
  // State per head: running max, weight sum, and the value accumulator split as the pages'
  // qdot pattern splits the dequantization: o[e] = sum_n p_n vs_n code_n[e] and pvb = sum_n
  // p_n vb_n (the slice lies in one group, so one bias per row), added together at the end.
  float mx[QC], lsum[QC], pvb[QC], o[QC][EL];
#pragma unroll
  for (int i = 0; i < QC; ++i) {
    mx[i] = -__builtin_inff();
    lsum[i] = 0.0f;
    pvb[i] = 0.0f;
#pragma unroll
    for (int e = 0; e < EL; ++e) o[i][e] = 0.0f;
  }
  // The wave's steps run in rounds of P: the rows of P steps are in flight at once.  A round
  // first takes the P steps' scores, then moves the running max once, then adds the P steps'
  // values; the next round's keys are issued once the scores are taken and its values once
  // the values are added (only when there is a next round: a uniform branch).  Every slot
  // is computed (steps past the block read its last row and are masked).  Nothing combines
  // a loaded value at issue, so no load is waited for before its round uses it.
  const int first = R * wv;   // the wave's first row in the block
  const int nsteps = first < nloc ? (nloc - first + kKvqWaves * R - 1) / (kKvqWaves * R) : 0;
  u4_t kw[P], vw[P];
  uint32_t ksr[P], kbr[P], vsr[P], vbr[P];   // the slice group's scale and bias bits
  auto row_of = [&](int q) __attribute__((always_inline)) {
    const int n = first + q * (kKvqWaves * R) + slot;
    return (uint32_t)(n < nloc ? n : nloc - 1);
  };
  auto issue_k = [&](int sl, int q) __attribute__((always_inline)) {
    const uint32_t r = row_of(q);
    kw[sl] = kc[r * LPR + j];
    ksr[sl] = ks[r * groups + gi];
    kbr[sl] = kb[r * groups + gi];
  };
  auto issue_v = [&](int sl, int q) __attribute__((always_inline)) {
    const uint32_t r = row_of(q);
    vw[sl] = vc[r * LPR + j];
    vsr[sl] = vs[r * groups + gi];
    vbr[sl] = vb[r * groups + gi];
  };
  auto sbf = [](uint32_t h) __attribute__((always_inline)) {
    return SBT == 1 ? (float)__builtin_bit_cast(_Float16, (uint16_t)h) : __builtin_bit_cast(float, h << 16);
  };
  // the slice's EL codes as floats (4-bit: the even and odd codes of a dword spread to bytes
  // first); each byte converts in one instruction
  auto codes = [&](const u4_t& w, float f[EL]) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if constexpr (BITS == 8) {
        bytes_to_float(w[d], f + 4 * d, 1);
      } else {
        bytes_to_float(w[d] & 0x0F0F0F0Fu, f + 8 * d, 2);          // even codes
        bytes_to_float((w[d] >> 4) & 0x0F0F0F0Fu, f + 8 * d + 1, 2);   // odd codes
      }
    }
  };
#pragma unroll
  for (int sl = 0; sl < P; ++sl) issue_k(sl, sl);
#pragma unroll
  for (int sl = 0; sl < P; ++sl) issue_v(sl, sl);
  __builtin_amdgcn_sched_barrier(0);
  for (int q0 = 0; q0 < nsteps; q0 += P) {
    const bool more = q0 + P < nsteps;
    float sc[P][QC];
    bool live[P];
#pragma unroll
    for (int sl = 0; sl < P; ++sl) {
      live[sl] = first + (q0 + sl) * (kKvqWaves * R) + slot < nloc;
      const float ksc = sbf(ksr[sl]), kbi = sbf(kbr[sl]);
      float kf[EL];
      codes(kw[sl], kf);
#pragma unroll
      for (int i = 0; i < QC; ++i) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < EL; ++e) dot = fmaf(qv[i][e], kf[e], dot);
        sc[sl][i] = lane_reduce<0, LB, false>(fmaf(ksc, dot, kbi * qsum[i]));   // the row's score on its LPR lanes
      }
    }
    if (more) {
#pragma unroll
      for (int sl = 0; sl < P; ++sl) issue_k(sl, q0 + P + sl);
    }
#pragma unroll
    for (int i = 0; i < QC; ++i) {
      float m = -__builtin_inff();
#pragma unroll
      for (int sl = 0; sl < P; ++sl) m = fmaxf(m, live[sl] ? sc[sl][i] : -__builtin_inff());
      const float mnew = fmaxf(mx[i], lane_reduce<LB, 6, true>(m));   // over the round's rows
      if (q0 != 0) {   // the first round's state is still zero: nothing to rescale
        // a round without live rows (mnew may still be -inf) leaves the state as it is
        const float f = mnew == -__builtin_inff() ? 1.0f : expf(mx[i] - mnew);
        lsum[i] *= f;
        pvb[i] *= f;
#pragma unroll
        for (int e = 0; e < EL; ++e) o[i][e] *= f;
      }
      mx[i] = mnew;
    }
#pragma unroll
    for (int sl = 0; sl < P; ++sl) {
      const float vsc = sbf(vsr[sl]), vbi = sbf(vbr[sl]);
      float vf[EL];
      codes(vw[sl], vf);
#pragma unroll
      for (int i = 0; i < QC; ++i) {
        const float p = live[sl] ? expf(sc[sl][i] - mx[i]) : 0.0f;
        lsum[i] += j == 0 ? p : 0.0f;   // one lane per row carries its weight
        pvb[i] = fmaf(p, vbi, pvb[i]);
        const float w = p * vsc;
#pragma unroll
        for (int e = 0; e < EL; ++e) o[i][e] = fmaf(w, vf[e], o[i][e]);
      }
    }
    if (more) {
#pragma unroll
      for (int sl = 0; sl < P; ++sl) issue_v(sl, q0 + P + sl);
    }
  }
#pragma unroll
  for (int i = 0; i < QC; ++i)
#pragma unroll
    for (int e = 0; e < EL; ++e) o[i][e] += pvb[i];
  // per head: sum over the row slots (lanes of one slice; a reduce-scatter leaves each lane
  // EL >> (6 - LB) of the slice's sums), then the wave's weight sum
  constexpr int KEEP = EL >> (6 - LB);
  static_assert(KEEP >= 1, "at least one sum per lane");
  const int sbase = j * EL + scatter_base<LB, EL>(lane);
#pragma unroll
  for (int i = 0; i < QC; ++i) {
    reduce_scatter<LB, EL>(o[i]);
    lsum[i] = lane_reduce<0, 6, false>(lsum[i]);
    if (lane == 0) {
      tg_max[i][wv] = mx[i];
      tg_sum[i][wv] = lsum[i];
    }
#pragma unroll
    for (int e = 0; e < KEEP; ++e) tg_o[i][wv * D + sbase + e] = o[i][e];
  }
  __syncthreads();
  if (wv < QC) {   // wave i merges head h0 + i
    const int i = wv;
    float M = tg_max[i][0];
    for (int w = 1; w < kKvqWaves; ++w) M = fmaxf(M, tg_max[i][w]);
    float wgt[kKvqWaves], S = 0.0f;
    for (int w = 0; w < kKvqWaves; ++w) {
      wgt[w] = tg_max[i][w] == -__builtin_inff() ? 0.0f : expf(tg_max[i][w] - M);   // a wave without rows
      S = fmaf(tg_sum[i][w], wgt[w], S);
    }
    const long base = ((long)(h0 + i) * a.G + g) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = lane * E + e;
      float v = 0.0f;
      for (int w = 0; w < kKvqWaves; ++w) v = fmaf(tg_o[i][w * D + d], wgt[w], v);
      a.opart[base + d] = v;
    }
    if (lane == 0) {
      a.stats[((long)(h0 + i) * a.G + g) * 2 + 0] = M;
      a.stats[((long)(h0 + i) * a.G + g) * 2 + 1] = S;
    }
  }
}

// A workgroup-wide reduction of one value per thread in a fixed order: a butterfly over the
// lane bits in each wave, then the four waves' results in wave order, read by every thread.
template <bool MAX>
__device__ __forceinline__ float merge_reduce(float v, float* part) {
  v = lane_reduce<0, 6, MAX>(v);
  __syncthreads();   // earlier readers of part are done
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = part[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = MAX ? fmaxf(r, part[w]) : r + part[w];
  return r;
}

// out[h, d] = sum_g opart[h, g, d] e^(M_g - M) / sum_g S_g e^(M_g - M).  One workgroup per
// (head, 64 columns); wave k of it sums its columns over the k-th quarter of the blocks
// (contiguous, in block order) and the quarters are added in order, so the result is the
// same on every run.  A thread's first kPrefetch partials and their block maxima are loaded
// before the statistics are reduced (M and the denominator: every thread takes blocks t,
// t + 256, ... in order, then merge_reduce), so the partials and the statistics arrive in
// one round of loads; the block weights e^(M_g - M) are formed in registers.
constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 64;
constexpr int kPrefetch = 16;
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const KvqParams a) {
  __shared__ float part[kMergeThreads];
  __shared__ float quarter[kMergeThreads / 64][kMergeCols];
  const int h = blockIdx.x, t = threadIdx.x, D = a.D, G = a.G;
  const int col = (int)blockIdx.y * kMergeCols + (t & 63), k = t >> 6;
  const int g_lo = (int)((long)G * k / 4), g_hi = (int)((long)G * (k + 1) / 4);   // this wave's blocks
  const float* st = a.stats + (long)h * G * 2;
  const float* op = a.opart + (long)h * G * D + col;
  float pre[kPrefetch], pm[kPrefetch];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) {
    const int g = min(g_lo + i, G - 1);
    pre[i] = op[(long)g * D];
    pm[i] = st[2 * g];
  }
  float m = -__builtin_inff();
  for (int g = t; g < G; g += kMergeThreads) m = fmaxf(m, st[2 * g]);
  const float M = merge_reduce<true>(m, part);
  float den = 0.0f;
  for (int g = t; g < G; g += kMergeThreads) den = fmaf(st[2 * g + 1], expf(st[2 * g] - M), den);
  const float den_all = merge_reduce<false>(den, part);
  float o = 0.0f;
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) o = g_lo + i < g_hi ? fmaf(pre[i], expf(pm[i] - M), o) : o;
#pragma unroll 8
  for (int g = g_lo + kPrefetch; g < g_hi; ++g) o = fmaf(op[(long)g * D], expf(st[2 * g] - M), o);
  quarter[k][t & 63] = o;
  __syncthreads();
  if (t < kMergeCols) {
    float v = quarter[0][t];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) v += quarter[w][t];
    v /= den_all;
    const long idx = (long)h * D + col;
    if (a.out_dtype == 0) static_cast<float*>(a.out)[idx] = v;
    else if (a.out_dtype == 1) static_cast<_Float16*>(a.out)[idx] = (_Float16)v;
    else static_cast<__bf16*>(a.out)[idx] = (__bf16)v;
  }
}

template <int BITS, int QC, int SBT, int QT>
hipError_t launch_block_qc(const KvqParams& a, hipStream_t s) {
  const dim3 grid(a.G, a.KV, (a.H / a.KV) / QC);
  switch (a.D) {
    case 64: hipLaunchKernelGGL((block_kernel<BITS, 64, QC, SBT, QT>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((block_kernel<BITS, 128, QC, SBT, QT>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL((block_kernel<BITS, 256, QC, SBT, QT>), grid, dim3(kKvqThreads), 0, s, a); break;
    case 512: hipLaunchKernelGGL((block_kernel<BITS, 512, QC, SBT, QT>), grid, dim3(kKvqThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Query heads per workgroup: two where the heads sharing a KV head pair up, else one.  The
// query's dtype is part of the instantiation (with it a runtime flag, every query element
// was widened both ways and one result selected: about 260 of a wave's 1,740 vector
// instructions; 13.75 -> 13.56 us on the 16-head, 8192-row call).
template <int BITS, int SBT>
hipError_t launch_block_sb(const KvqParams& a, hipStream_t s) {
  const bool pair = (a.H / a.KV) % 2 == 0;
  if (a.q_dtype == 1) return pair ? launch_block_qc<BITS, 2, SBT, 1>(a, s) : launch_block_qc<BITS, 1, SBT, 1>(a, s);
  return pair ? launch_block_qc<BITS, 2, SBT, 2>(a, s) : launch_block_qc<BITS, 1, SBT, 2>(a, s);
}
template <int BITS>
hipError_t launch_block(const KvqParams& a, hipStream_t s) {
  return a.sb_dtype == 1 ? launch_block_sb<BITS, 1>(a, s) : launch_block_sb<BITS, 2>(a, s);
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
  hipLaunchKernelGGL(merge_kernel, dim3(a.H, a.D / kMergeCols), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlin
