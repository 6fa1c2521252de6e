// libqlin host side: argument validation, variant selection, launches, hipGraph chains.
// The ABI and its conventions are documented in include/qlin.h.
#include "qlin.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>

#include "qlin_fused.h"
#include "qlin_internal.h"

namespace {

std::atomic<int64_t> g_dispatch[10];

constexpr int64_t kMaxK = int64_t(1) << 20;   // keeps every in-kernel row offset within int range
constexpr int64_t kMaxN = int64_t(1) << 28;
constexpr int kMaxT = 32;
constexpr int kMaxPositions = 32;    // attend: cached + new positions (one key per lane of a half wave)
constexpr int kMaxHeads = 1 << 16;
constexpr int kMaxHeadDim = 512;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t dtype_size(int d) { return d == QLIN_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || !an || !bn) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

qlin_status check_weight(const qlin_weight* w, int x_dtype, bool nonempty) {
  if (!w) return QLIN_ERR_NULL;
  if (w->bits != 4 && w->bits != 8 && w->bits != 16) return QLIN_ERR_BITS;
  if (w->bits != 16 && w->group_size != 64) return QLIN_ERR_BITS;
  if (w->K <= 0 || w->K % 64 != 0 || w->K > kMaxK) return QLIN_ERR_SHAPE;
  if (w->N < 0 || w->N > kMaxN) return QLIN_ERR_SHAPE;
  if (w->bits == 16) {
    if (w->dtype != x_dtype) return QLIN_ERR_DTYPE;
  } else if (w->dtype != QLIN_F16) {
    return QLIN_ERR_DTYPE;
  }
  if (nonempty && w->N > 0) {
    if (!w->data) return QLIN_ERR_NULL;
    if (!aligned(w->data, 16)) return QLIN_ERR_ALIGN;
    if (w->bits != 16) {
      if (!w->scales || !w->biases) return QLIN_ERR_NULL;
      if (!aligned(w->scales, 2) || !aligned(w->biases, 2)) return QLIN_ERR_ALIGN;
    }
  }
  return QLIN_OK;
}

qlin_status validate(const void* x, int x_dtype, int32_t T, const qlin_weight* w, const qlin_weight* up,
                     const qlin_ln* ln, int act, const void* res, const void* add, const void* y, int y_dtype) {
  if (!w) return QLIN_ERR_NULL;
  if (x_dtype != QLIN_F16 && x_dtype != QLIN_BF16) return QLIN_ERR_DTYPE;
  if (y_dtype != QLIN_F32 && y_dtype != QLIN_F16 && y_dtype != QLIN_BF16) return QLIN_ERR_DTYPE;
  if (T < 0 || T > kMaxT) return QLIN_ERR_SHAPE;
  if (act != QLIN_ACT_NONE && act != QLIN_ACT_GELU) return QLIN_ERR_ARG;
  const bool nonempty = T > 0;
  qlin_status st = check_weight(w, x_dtype, nonempty);
  if (st != QLIN_OK) return st;
  if (up) {
    st = check_weight(up, x_dtype, nonempty);
    if (st != QLIN_OK) return st;
    if (up->bits != w->bits) return QLIN_ERR_BITS;
    if (up->dtype != w->dtype) return QLIN_ERR_DTYPE;
    if (up->N != w->N || up->K != w->K) return QLIN_ERR_SHAPE;
    if (act != QLIN_ACT_NONE || res || add) return QLIN_ERR_ARG;
  }
  if (ln) {
    if (!(ln->eps >= 0.0f) || !std::isfinite(ln->eps)) return QLIN_ERR_ARG;
  }
  if (!nonempty || w->N == 0) return QLIN_OK;   // empty: a valid no-op
  if (!x || !y) return QLIN_ERR_NULL;
  if (!aligned(x, 16)) return QLIN_ERR_ALIGN;
  if (!aligned(y, dtype_size(y_dtype))) return QLIN_ERR_ALIGN;
  if (ln) {
    if (!ln->gamma || !ln->beta) return QLIN_ERR_NULL;
    if (!aligned(ln->gamma, 16) || !aligned(ln->beta, 16)) return QLIN_ERR_ALIGN;
  }
  if (res && !aligned(res, 2)) return QLIN_ERR_ALIGN;
  if (add && !aligned(add, 2)) return QLIN_ERR_ALIGN;
  const size_t ybytes = (size_t)T * (size_t)w->N * dtype_size(y_dtype);
  if (overlaps(y, ybytes, x, (size_t)T * (size_t)w->K * 2)) return QLIN_ERR_ARG;
  if (overlaps(y, ybytes, res, (size_t)T * (size_t)w->N * 2)) return QLIN_ERR_ARG;
  return QLIN_OK;
}

// Compute units of the current device, queried once per device.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Which kernel family serves quantized calls: 0 the int8 streaming kernel where its shape
// rules admit the call (else the general kernel), 1 always the general kernel, 2 the
// vector-ALU kernel where it applies.
std::atomic<int> g_path{0};

// Polls a merge wait of the general kernel makes before it gives up, and the device counter
// of the waits that gave up (one per GPU; its address looked up once per device).
std::atomic<int> g_merge_spin{qlin::kSpinMax};
static __device__ unsigned int g_merge_timeouts;

hipError_t merge_timeouts_ptr(unsigned int** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static unsigned int* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_merge_timeouts));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<unsigned int*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// The int8 streaming kernel (qlin_s8.h) for 4- and 8-bit codes.  Returns false when its
// shape rules do not admit the call (the general kernel takes it then).
bool try_s8(const void* x, int x_dtype, int32_t T, const qlin_weight* w, const qlin_weight* up, const qlin_ln* ln,
            int act, const void* res, const void* add, void* y, int y_dtype, hipStream_t stream, hipError_t* err) {
  using namespace qlin;
  if (g_path.load(std::memory_order_relaxed) == 1) return false;
  if (w->bits != 4 && w->bits != 8) return false;
  if (up && ln) return false;
  const int G = (int)(w->K / 64);
  for (const qlin_weight* q : {w, up}) {
    if (q && (!aligned(q->scales, 16) || !aligned(q->biases, 16))) return false;
  }
  const int R = T + (ln ? 2 : 0);
  const int mt = R <= 4 ? 1 : (R <= 8 ? 2 : (R <= 12 ? 3 : 9));
  const int ntiles = (int)(up ? (w->N + 7) / 8 : (w->N + 15) / 16);
  // The window of K per wave (a power of two, >= 2 groups): up to 8 waves per workgroup, two
  // per SIMD, so that one wave's arithmetic runs while the other waits for its tile (on
  // the SwiGLU shape 14.4 us against 15.5 with one wave of twice the window per SIMD).
  auto window = [&](int waves) { return pow2_ceil(G <= 2 * waves ? 2 : (G + waves - 1) / waves); };
  const int bits = w->bits;
  const bool lnb = ln != nullptr;
  auto usable = [&](int g) { return g <= 32 && G % (g < 8 ? g : 8) == 0 && s8::max_tiles(bits, lnb, mt, g) > 0; };
  int gw = window(8);
  if (!usable(gw)) return false;
  // One tile per workgroup: up to 16 waves where the shorter windows give more than 8 of
  // them, so that more of the rows' loads are in flight at once.
  if (ntiles <= cu_count()) {
    const int g16 = window(16);
    if ((G + g16 - 1) / g16 > 8 && s8::wide_ok(bits, lnb, mt, g16) && G % (g16 < 8 ? g16 : 8) == 0) gw = g16;
  }
  const int dm = (G + gw - 1) / gw > 8 ? 1 : s8::max_tiles(bits, lnb, mt, gw);
  S8Launch a{};
  a.x = x;
  a.w0 = w->data; a.s0 = w->scales; a.b0 = w->biases;
  if (up) { a.p1 = up->data; a.p2 = up->scales; a.p3 = up->biases; }
  else if (ln) { a.p1 = ln->gamma; a.p2 = ln->beta; a.p3 = nullptr; }
  a.K = (int)w->K; a.T = T; a.N = (int)w->N; a.x_bf16 = x_dtype == QLIN_BF16 ? 1 : 0;
  a.gateup = up ? 1 : 0; a.ln = ln ? 1 : 0; a.bits = w->bits;
  a.y = y; a.res = res; a.add = add; a.eps = ln ? ln->eps : 0.0f; a.y_dtype = y_dtype; a.act = act;
  a.MT = mt; a.GWM = gw; a.waves = (G + gw - 1) / gw;
  int tpw = (ntiles + cu_count() - 1) / cu_count();
  if (tpw > dm) tpw = dm;
  a.grid = (ntiles + tpw - 1) / tpw;
  a.D = (ntiles + a.grid - 1) / a.grid;   // tiles of the fullest workgroup
  // the shape rides in the top 16 bits of the pointer arguments (qlin_s8.h)
  if (a.grid > 0xFFFF) return false;
  for (const void* q : {a.x, a.w0, a.s0, a.b0, a.p1, a.p2, a.p3}) {
    if ((reinterpret_cast<uintptr_t>(q) >> s8::kTagShift) != 0) return false;
  }
  using L = hipError_t (*)(const S8Launch&, hipStream_t);
  static const L table[2][2][2] = {   // [8-bit][LayerNorm][bf16 activations]
      {{launch_s8_q4_ln0_f16, launch_s8_q4_ln0_bf16}, {launch_s8_q4_ln1_f16, launch_s8_q4_ln1_bf16}},
      {{launch_s8_q8_ln0_f16, launch_s8_q8_ln0_bf16}, {launch_s8_q8_ln1_f16, launch_s8_q8_ln1_bf16}}};
  *err = table[w->bits == 8][ln ? 1 : 0][a.x_bf16 ? 1 : 0](a, stream);
  return true;
}

// The vector-ALU kernel (qlin_valu.h) for 4- and 8-bit codes and T <= 4, when selected.
// Returns false when it does not take the call.
bool try_valu(const void* x, int x_dtype, int32_t T, const qlin_weight* w, const qlin_weight* up, const qlin_ln* ln,
              int act, const void* res, const void* add, void* y, int y_dtype, hipStream_t stream, hipError_t* err) {
  using namespace qlin;
  if (g_path.load(std::memory_order_relaxed) != 2) return false;
  const bool dense16 = w->bits == 16 && w->dtype == QLIN_F16 && x_dtype == QLIN_F16;
  if ((w->bits != 4 && w->bits != 8 && !dense16) || T > 4 || (up && ln)) return false;
  const int tt = T == 1 ? 1 : (T == 2 ? 2 : 4);
  const int K = (int)w->K;
  int lpr = 0, waves = 0;
  for (int l : {16, 32}) {
    const int maxw = (l == 16 && !ln) ? 16 : 8;
    const int wv = (K + 16 * l - 1) / (16 * l);
    if (wv <= maxw && !(l == 32 && ln && tt == 4)) { lpr = l; waves = wv; break; }
  }
  if (lpr == 0) return false;
  const int ntiles = (int)(up ? (w->N + 7) / 8 : (w->N + 15) / 16);
  int tpw = (ntiles + cu_count() - 1) / cu_count();
  if (tpw > 8) tpw = 8;
  S8Launch a{};
  a.x = x;
  a.w0 = w->data; a.s0 = w->scales; a.b0 = w->biases;
  if (up) { a.p1 = up->data; a.p2 = up->scales; a.p3 = up->biases; }
  else if (ln) { a.p1 = ln->gamma; a.p2 = ln->beta; a.p3 = nullptr; }
  a.K = K; a.T = T; a.N = (int)w->N; a.x_bf16 = x_dtype == QLIN_BF16 ? 1 : 0;
  a.gateup = up ? 1 : 0; a.ln = ln ? 1 : 0; a.bits = w->bits;
  a.y = y; a.res = res; a.add = add; a.eps = ln ? ln->eps : 0.0f; a.y_dtype = y_dtype; a.act = act;
  a.MT = tt; a.GWM = lpr; a.waves = waves;
  a.grid = (ntiles + tpw - 1) / tpw;
  a.D = (ntiles + a.grid - 1) / a.grid;
  if (a.grid > 0xFFFF) return false;
  for (const void* q : {a.x, a.w0, a.s0, a.b0, a.p1, a.p2, a.p3}) {
    if ((reinterpret_cast<uintptr_t>(q) >> s8::kTagShift) != 0) return false;
  }
  *err = w->bits == 4 ? launch_valu_q4(a, stream) : w->bits == 8 ? launch_valu_q8(a, stream) : launch_valu_f16(a, stream);
  return true;
}

qlin_status launch(const void* x, int x_dtype, int32_t T, const qlin_weight* w, const qlin_weight* up,
                   const qlin_ln* ln, int act, const void* res, const void* add, void* y, int y_dtype,
                   hipStream_t stream) {
  using namespace qlin;
  {
    hipError_t e = hipSuccess;
    if (try_valu(x, x_dtype, T, w, up, ln, act, res, add, y, y_dtype, stream, &e)) {
      if (e != hipSuccess) return QLIN_ERR_HIP;
      g_dispatch[up ? 1 : 0].fetch_add(1, std::memory_order_relaxed);
      g_dispatch[9].fetch_add(1, std::memory_order_relaxed);
      return QLIN_OK;
    }
    if (try_s8(x, x_dtype, T, w, up, ln, act, res, add, y, y_dtype, stream, &e)) {
      if (e != hipSuccess) return QLIN_ERR_HIP;
      g_dispatch[up ? 1 : 0].fetch_add(1, std::memory_order_relaxed);
      g_dispatch[8].fetch_add(1, std::memory_order_relaxed);
      return QLIN_OK;
    }
  }
  LinParams p{};
  p.x = x; p.x_dtype = x_dtype; p.T = T; p.K = (int)w->K; p.N = (int)w->N;
  p.w[0] = w->data; p.sc[0] = static_cast<const uint16_t*>(w->scales); p.bi[0] = static_cast<const uint16_t*>(w->biases);
  p.gateup = up != nullptr;
  if (up) { p.w[1] = up->data; p.sc[1] = static_cast<const uint16_t*>(up->scales); p.bi[1] = static_cast<const uint16_t*>(up->biases); }
  else { p.w[1] = p.w[0]; p.sc[1] = p.sc[0]; p.bi[1] = p.bi[0]; }
  p.ln = ln != nullptr;
  p.gamma = ln ? ln->gamma : nullptr; p.beta = ln ? ln->beta : nullptr; p.eps = ln ? ln->eps : 0.0f;
  const bool bf16op = w->bits == 16 && w->dtype == QLIN_BF16;
  if (bf16op) {            // dense bf16 weights: bf16 operands, exact 1- or 3-term activations
    // (bf16 x is one bf16 term; fp16 x and LN outputs need three)
    p.terms = (p.ln || x_dtype == QLIN_F16) ? 3 : 1; p.scale_act = 0; p.scale_gb = 0;
  } else {                 // fp16 operands: 1 term without LN, else 2; activation rows are always
    // scaled by a power of two into [2^14, 2^15) at their maximum, so that small values stay
    // normal (the matrix cores lose precision on subnormal inputs next to larger products)
    p.terms = p.ln ? 2 : 1;
    p.scale_act = 1;
    p.scale_gb = (p.ln && x_dtype == QLIN_BF16) ? 1 : 0;
  }
  p.act = act; p.res = res; p.add = add; p.y = y; p.y_dtype = y_dtype;
  p.spin = g_merge_spin.load(std::memory_order_relaxed);
  if (merge_timeouts_ptr(&p.timeouts) != hipSuccess) return QLIN_ERR_HIP;
  p.rows = act_rows(T, p.terms, p.ln);
  const int mt = (p.rows + 15) / 16;
  const int64_t row_bytes = w->K * w->bits / 8;
  p.steps = (int)((row_bytes + 63) / 64);
  p.chunk_steps = fused_chunk_steps(w->bits, mt, T, p.ln, p.rows, w->K);
  p.ntiles = (int)(up ? (w->N + 7) / 8 : (w->N + 15) / 16);
  const int grid = p.ntiles < cu_count() ? p.ntiles : cu_count();
  const size_t lds = fused_lds_bytes(w->bits, p.rows, p.chunk_steps, w->K, mt);
  hipError_t e;
  if (w->bits == 4) e = launch_fused_q4(p, mt, grid, lds, stream);
  else if (w->bits == 8) e = launch_fused_q8(p, mt, grid, lds, stream);
  else if (bf16op) e = launch_fused_bf16(p, mt, grid, lds, stream);
  else e = launch_fused_f16(p, mt, grid, lds, stream);
  if (e != hipSuccess) return QLIN_ERR_HIP;
  g_dispatch[up ? 1 : 0].fetch_add(1, std::memory_order_relaxed);
  return QLIN_OK;
}

}  // namespace

namespace qlin {
static int step_k(int bits) { return bits == 4 ? Fmt<4>::kStepK : (bits == 8 ? Fmt<8>::kStepK : Fmt<16>::kStepK); }
static long chunk_k(int bits, int cs, long K) { const long kc = (long)cs * step_k(bits); return kc < K ? kc : K; }

int fused_chunk_steps(int bits, int mt, int T, int ln, int rows, long K) {
  const int mfma = bits == 4 ? Fmt<4>::kMfma : (bits == 8 ? Fmt<8>::kMfma : Fmt<16>::kMfma);
  int cs = kWaves * max_steps_for(mfma, mt);
  const long srows = T + (ln ? 2 : 0);
  for (; cs > 1; --cs) {
    const long kc = chunk_k(bits, cs, K);
    const long pieces = srows * (kc / 8);   // staged 8-element pieces, shared by all threads
    if (pieces <= (long)kThreads * kPieceMax && lds_bytes_for(rows, (int)kc, mt) <= kLdsMax) break;
  }
  return cs;
}

size_t fused_lds_bytes(int bits, int rows, int chunk_steps, long K, int mt) {
  return (size_t)lds_bytes_for(rows, (int)chunk_k(bits, chunk_steps, K), mt);
}
}  // namespace qlin

struct qlin_chain {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int32_t n = 0;
};

extern "C" {

qlin_status qlin_check(const void* x, qlin_dtype x_dtype, int32_t T, const qlin_weight* w, const qlin_weight* up,
                       const qlin_ln* ln, qlin_act act, const void* residual, const void* add, const void* y,
                       qlin_dtype y_dtype) {
  return validate(x, x_dtype, T, w, up, ln, act, residual, add, y, y_dtype);
}

qlin_status qlin_linear(const void* x, qlin_dtype x_dtype, int32_t T, const qlin_weight* w, const qlin_ln* ln,
                        qlin_act act, const void* residual, const void* add, void* y, qlin_dtype y_dtype,
                        void* stream) {
  const qlin_status st = validate(x, x_dtype, T, w, nullptr, ln, act, residual, add, y, y_dtype);
  if (st != QLIN_OK) return st;
  if (T == 0 || w->N == 0) return QLIN_OK;
  return launch(x, x_dtype, T, w, nullptr, ln, act, residual, add, y, y_dtype, static_cast<hipStream_t>(stream));
}

qlin_status qlin_gateup_swiglu(const void* x, qlin_dtype x_dtype, int32_t T, const qlin_weight* gate,
                               const qlin_weight* up, const qlin_ln* ln, void* y, qlin_dtype y_dtype, void* stream) {
  if (!up) return QLIN_ERR_NULL;
  const qlin_status st = validate(x, x_dtype, T, gate, up, ln, QLIN_ACT_NONE, nullptr, nullptr, y, y_dtype);
  if (st != QLIN_OK) return st;
  if (T == 0 || gate->N == 0) return QLIN_OK;
  return launch(x, x_dtype, T, gate, up, ln, QLIN_ACT_NONE, nullptr, nullptr, y, y_dtype,
                static_cast<hipStream_t>(stream));
}

qlin_status qlin_pack_affine(const float* w, int64_t N, int64_t K, int32_t bits, int32_t group_size, uint32_t* codes,
                             void* scales, void* biases, qlin_dtype sb_dtype, int32_t* nonfinite_flag, void* stream) {
  if (bits != 4 && bits != 8) return QLIN_ERR_BITS;
  if (group_size != 64) return QLIN_ERR_BITS;
  if (sb_dtype != QLIN_F16) return QLIN_ERR_DTYPE;
  if (N < 0 || N > kMaxN || K <= 0 || K % 64 != 0 || K > kMaxK) return QLIN_ERR_SHAPE;
  if (N == 0) return QLIN_OK;
  if (!w || !codes || !scales || !biases) return QLIN_ERR_NULL;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(biases, 2)) return QLIN_ERR_ALIGN;
  if (nonfinite_flag && !aligned(nonfinite_flag, 4)) return QLIN_ERR_ALIGN;
  const hipError_t e = qlin::launch_pack(w, N, K, bits, codes, static_cast<uint16_t*>(scales),
                                         static_cast<uint16_t*>(biases), nonfinite_flag, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return QLIN_ERR_HIP;
  g_dispatch[2].fetch_add(1, std::memory_order_relaxed);
  return QLIN_OK;
}

qlin_status qlin_unpack_affine(const qlin_weight* w, float* out, void* stream) {
  if (!w) return QLIN_ERR_NULL;
  const int x_dtype = w->bits == 16 ? w->dtype : QLIN_F16;
  if (w->bits == 16 && w->dtype != QLIN_F16 && w->dtype != QLIN_BF16) return QLIN_ERR_DTYPE;
  const qlin_status st = check_weight(w, x_dtype, true);
  if (st != QLIN_OK) return st;
  if (w->N == 0) return QLIN_OK;
  if (!out) return QLIN_ERR_NULL;
  if (!aligned(out, 4)) return QLIN_ERR_ALIGN;
  const hipError_t e = qlin::launch_unpack(w->data, static_cast<const uint16_t*>(w->scales),
                                           static_cast<const uint16_t*>(w->biases), w->bits, w->dtype, w->N, w->K, out,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return QLIN_ERR_HIP;
  g_dispatch[3].fetch_add(1, std::memory_order_relaxed);
  return QLIN_OK;
}

qlin_status qlin_attend_check(const void* qkv, const void* kv, qlin_dtype dtype, int32_t P, int32_t T,
                              int32_t heads, int32_t head_dim, int32_t last, const void* out, qlin_dtype out_dtype,
                              const void* kv_out) {
  if (dtype != QLIN_F16 && dtype != QLIN_BF16) return QLIN_ERR_DTYPE;
  if (out_dtype != QLIN_F32 && out_dtype != QLIN_F16 && out_dtype != QLIN_BF16) return QLIN_ERR_DTYPE;
  if (T < 1 || P < 0 || P > kMaxPositions - T) return QLIN_ERR_SHAPE;
  if (heads < 1 || heads > kMaxHeads) return QLIN_ERR_SHAPE;
  if (head_dim < 16 || head_dim > kMaxHeadDim || head_dim % 16 != 0) return QLIN_ERR_SHAPE;
  if (last != 0 && last != 1) return QLIN_ERR_ARG;
  if (!qkv || !out || !kv_out || (P > 0 && !kv)) return QLIN_ERR_NULL;
  if (!aligned(qkv, 16) || !aligned(kv_out, 16) || (P > 0 && !aligned(kv, 16))) return QLIN_ERR_ALIGN;
  if (!aligned(out, dtype_size(out_dtype))) return QLIN_ERR_ALIGN;
  const size_t D = (size_t)heads * (size_t)head_dim;
  const size_t qkv_bytes = (size_t)T * 3 * D * 2, kv_bytes = P > 0 ? 2 * (size_t)P * D * 2 : 0;
  const size_t kv_out_bytes = 2 * (size_t)(P + T) * D * 2, out_bytes = (last ? 1 : (size_t)T) * D * dtype_size(out_dtype);
  if (overlaps(kv_out, kv_out_bytes, qkv, qkv_bytes) || overlaps(kv_out, kv_out_bytes, kv, kv_bytes)) return QLIN_ERR_ARG;
  if (overlaps(out, out_bytes, qkv, qkv_bytes) || overlaps(out, out_bytes, kv, kv_bytes) ||
      overlaps(out, out_bytes, kv_out, kv_out_bytes))
    return QLIN_ERR_ARG;
  return QLIN_OK;
}

qlin_status qlin_attend(const void* qkv, const void* kv, qlin_dtype dtype, int32_t P, int32_t T, int32_t heads,
                        int32_t head_dim, int32_t last, void* out, qlin_dtype out_dtype, void* kv_out, void* stream) {
  const qlin_status st = qlin_attend_check(qkv, kv, dtype, P, T, heads, head_dim, last, out, out_dtype, kv_out);
  if (st != QLIN_OK) return st;
  qlin::AttendParams a{};
  a.qkv = qkv; a.kv = P > 0 ? kv : nullptr; a.out = out; a.kv_out = kv_out;
  a.dtype = dtype; a.out_dtype = out_dtype;
  a.H = heads; a.HD = head_dim; a.P = P; a.T = T; a.last = last;
  a.scale = (float)(1.0 / std::sqrt((double)head_dim));
  if (qlin::launch_attend(a, static_cast<hipStream_t>(stream)) != hipSuccess) return QLIN_ERR_HIP;
  g_dispatch[4].fetch_add(1, std::memory_order_relaxed);
  return QLIN_OK;
}

qlin_status qlin_chain_create(const qlin_pass* passes, int32_t n_passes, qlin_dtype x_dtype, qlin_dtype y_dtype,
                              void* capture_stream, qlin_chain** out) {
  if (!out) return QLIN_ERR_NULL;
  *out = nullptr;
  if (!passes) return QLIN_ERR_NULL;
  if (n_passes < 1) return QLIN_ERR_ARG;
  if (!capture_stream) return QLIN_ERR_ARG;   // the null stream cannot be captured
  for (int32_t i = 0; i < n_passes; ++i) {
    const qlin_pass& q = passes[i];
    qlin_ln ln{q.ln_gamma, q.ln_beta, q.ln_eps};
    const qlin_status st = validate(q.x, x_dtype, q.T, &q.w, nullptr, q.ln_gamma ? &ln : nullptr, q.act, q.residual,
                                    q.add, q.y, y_dtype);
    if (st != QLIN_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(capture_stream);
  if (hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed) != hipSuccess) return QLIN_ERR_HIP;
  qlin_status st = QLIN_OK;
  for (int32_t i = 0; i < n_passes && st == QLIN_OK; ++i) {
    const qlin_pass& q = passes[i];
    qlin_ln ln{q.ln_gamma, q.ln_beta, q.ln_eps};
    st = qlin_linear(q.x, x_dtype, q.T, &q.w, q.ln_gamma ? &ln : nullptr, static_cast<qlin_act>(q.act), q.residual,
                     q.add, q.y, y_dtype, capture_stream);
  }
  hipGraph_t graph = nullptr;
  const hipError_t ee = hipStreamEndCapture(s, &graph);
  if (st != QLIN_OK || ee != hipSuccess || !graph) {
    if (graph) hipGraphDestroy(graph);
    return st != QLIN_OK ? st : QLIN_ERR_HIP;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    hipGraphDestroy(graph);
    return QLIN_ERR_HIP;
  }
  qlin_chain* c = new (std::nothrow) qlin_chain;
  if (!c) {
    hipGraphExecDestroy(exec);
    hipGraphDestroy(graph);
    return QLIN_ERR_HIP;
  }
  c->graph = graph; c->exec = exec; c->n = n_passes;
  *out = c;
  return QLIN_OK;
}

qlin_status qlin_chain_launch(qlin_chain* chain, void* stream) {
  if (!chain) return QLIN_ERR_NULL;
  if (hipGraphLaunch(chain->exec, static_cast<hipStream_t>(stream)) != hipSuccess) return QLIN_ERR_HIP;
  return QLIN_OK;
}

int32_t qlin_chain_passes(const qlin_chain* chain) { return chain ? chain->n : 0; }

void qlin_chain_destroy(qlin_chain* chain) {
  if (!chain) return;
  if (chain->exec) hipGraphExecDestroy(chain->exec);
  if (chain->graph) hipGraphDestroy(chain->graph);
  delete chain;
}

qlin_status qlin_mlp(const void* x, qlin_dtype x_dtype, int32_t T, const qlin_weight* gate, const qlin_weight* up,
                     const qlin_weight* down, const qlin_ln* ln, const void* residual, void* h, void* y,
                     qlin_dtype y_dtype, void* stream) {
  if (!gate || !up || !down) return QLIN_ERR_NULL;
  qlin_status st = validate(x, x_dtype, T, gate, up, ln, QLIN_ACT_NONE, nullptr, nullptr, h, x_dtype);
  if (st != QLIN_OK) return st;
  if (down->K != gate->N) return QLIN_ERR_SHAPE;
  st = validate(h, x_dtype, T, down, nullptr, nullptr, QLIN_ACT_NONE, residual, nullptr, y, y_dtype);
  if (st != QLIN_OK) return st;
  if (T == 0 || down->N == 0) return QLIN_OK;   // empty y: a valid no-op (I = down->K >= 64)
  const size_t hbytes = (size_t)T * (size_t)gate->N * 2;
  const size_t ybytes = (size_t)T * (size_t)down->N * dtype_size(y_dtype);
  if (overlaps(h, hbytes, x, (size_t)T * (size_t)gate->K * 2)) return QLIN_ERR_ARG;
  if (overlaps(h, hbytes, residual, (size_t)T * (size_t)down->N * 2)) return QLIN_ERR_ARG;
  if (overlaps(h, hbytes, y, ybytes)) return QLIN_ERR_ARG;
  for (const qlin_weight* w : {gate, up, down}) {
    const size_t wb = (size_t)w->N * (size_t)w->K * (size_t)w->bits / 8;
    if (overlaps(h, hbytes, w->data, wb)) return QLIN_ERR_ARG;
    if (w->bits != 16) {
      const size_t sb = (size_t)w->N * (size_t)(w->K / 64) * 2;
      if (overlaps(h, hbytes, w->scales, sb) || overlaps(h, hbytes, w->biases, sb)) return QLIN_ERR_ARG;
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch(x, x_dtype, T, gate, up, ln, QLIN_ACT_NONE, nullptr, nullptr, h, x_dtype, s);
  if (st != QLIN_OK) return st;
  return launch(h, x_dtype, T, down, nullptr, nullptr, QLIN_ACT_NONE, residual, nullptr, y, y_dtype, s);
}

qlin_status qlin_stream_read_config(const void* buf, int64_t bytes, uint32_t* partial, int32_t blocks, int32_t unroll,
                                   int32_t nontemporal, void* stream) {
  if (!buf || !partial) return QLIN_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0) return QLIN_ERR_SHAPE;
  if (blocks < 1 || blocks > QLIN_STREAM_READ_BLOCKS) return QLIN_ERR_ARG;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16) return QLIN_ERR_ARG;
  if (nontemporal != 0 && nontemporal != 1) return QLIN_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(partial) & 3u) != 0)
    return QLIN_ERR_ALIGN;
  if (qlin::launch_stream_read(buf, bytes, partial, blocks, unroll, nontemporal != 0,
                               static_cast<hipStream_t>(stream)) != hipSuccess)
    return QLIN_ERR_HIP;
  g_dispatch[5].fetch_add(1, std::memory_order_relaxed);
  return QLIN_OK;
}

qlin_status qlin_stream_read(const void* buf, int64_t bytes, uint32_t* partial, void* stream) {
  const int cus = cu_count();
  return qlin_stream_read_config(buf, bytes, partial, cus < QLIN_STREAM_READ_BLOCKS ? cus : QLIN_STREAM_READ_BLOCKS,
                                 4, 1, stream);
}

qlin_status qlin_sample(const void* logits, qlin_dtype logit_dtype, int32_t n, const float* gumbel, float inv_temp,
                        int32_t top_k, const void* table, const void* prefix, int32_t n_prev, int32_t D,
                        qlin_dtype emb_dtype, void* out, int32_t* code, void* stream) {
  if (!logits || !gumbel || !code) return QLIN_ERR_NULL;
  if (logit_dtype != QLIN_F32 && logit_dtype != QLIN_F16 && logit_dtype != QLIN_BF16) return QLIN_ERR_DTYPE;
  if (emb_dtype != QLIN_F32 && emb_dtype != QLIN_F16 && emb_dtype != QLIN_BF16) return QLIN_ERR_DTYPE;
  if (n < 1 || n > qlin::kSampleMaxCodes || top_k < 1 || top_k > n) return QLIN_ERR_SHAPE;
  if (n_prev < 0 || n_prev > (1 << 20)) return QLIN_ERR_SHAPE;
  if (!(inv_temp > 0.0f) || !std::isfinite(inv_temp)) return QLIN_ERR_ARG;
  const size_t ls = dtype_size(logit_dtype), es = dtype_size(emb_dtype);
  if (!aligned(logits, ls) || !aligned(gumbel, 4) || !aligned(code, 4)) return QLIN_ERR_ALIGN;
  const bool rows = table != nullptr || n_prev > 0;
  if (rows) {
    if (D < 1 || ((size_t)D * es) % 16 != 0 || D > (1 << 20)) return QLIN_ERR_SHAPE;
    if (!out || (n_prev > 0 && !prefix)) return QLIN_ERR_NULL;
    if (!aligned(out, 16) || (table && !aligned(table, 16)) || (n_prev > 0 && !aligned(prefix, 16)))
      return QLIN_ERR_ALIGN;
  }
  const size_t row = (size_t)D * es;
  const size_t outb = rows ? (size_t)(n_prev + (table ? 1 : 0)) * row : 0;
  const bool in_place = n_prev > 0 && out == prefix;
  if (rows) {
    if (n_prev > 0 && !in_place && overlaps(out, outb, prefix, (size_t)n_prev * row)) return QLIN_ERR_ARG;
    if (in_place && table && overlaps(static_cast<const char*>(out) + (size_t)n_prev * row, row, prefix,
                                      (size_t)n_prev * row)) return QLIN_ERR_ARG;
    if (table && overlaps(out, outb, table, (size_t)n * row)) return QLIN_ERR_ARG;
    if (overlaps(out, outb, logits, (size_t)n * ls) || overlaps(out, outb, gumbel, (size_t)n * 4) ||
        overlaps(out, outb, code, 4)) return QLIN_ERR_ARG;
  }
  if (overlaps(code, 4, logits, (size_t)n * ls) || overlaps(code, 4, gumbel, (size_t)n * 4)) return QLIN_ERR_ARG;
  qlin::SampleParams a{};
  a.logits = logits; a.logit_dtype = logit_dtype; a.n = n; a.gumbel = gumbel; a.inv_temp = inv_temp;
  a.top_k = top_k; a.table = table; a.prefix = prefix; a.n_prev = rows ? n_prev : 0; a.D = rows ? D : 0;
  a.es = (int)es; a.out = out; a.code = code; a.copy_prefix = (n_prev > 0 && !in_place) ? 1 : 0;
  if (qlin::launch_sample(a, static_cast<hipStream_t>(stream)) != hipSuccess) return QLIN_ERR_HIP;
  g_dispatch[6].fetch_add(1, std::memory_order_relaxed);
  return QLIN_OK;
}

namespace {
// Rows per block of the quantized-KV decode: 256 (a workgroup of eight waves per 256 rows
// and head pair), 512 once the blocks would pass 8192 per head (bounding the workspace at
// large n_rows).
int kvq_block(int32_t n_rows) { return n_rows <= 256 * 8192 ? 256 : 512; }
}  // namespace

int64_t qlin_kvq_decode_workspace(int32_t heads, int32_t n_rows, int32_t head_dim) {
  if (heads < 1 || n_rows < 1 || head_dim < 1) return 0;
  const int64_t G = (n_rows + kvq_block(n_rows) - 1) / kvq_block(n_rows);
  return (int64_t)heads * G * ((int64_t)head_dim + 2) * 4;
}

namespace {
// Checks and launch shared by qlin_kvq_decode and qlin_kvq_decode_noalloc.  ws == null asks
// for the library's static scratch (the no-allocation entry point); otherwise ws holds
// ws_bytes bytes of caller workspace.
qlin_status kvq_run(const void* q, qlin_dtype q_dtype, int32_t heads, int32_t kv_heads, int32_t n_rows,
                    int32_t head_dim, int32_t group_size, int32_t bits, const uint32_t* k_codes,
                    const void* k_scales, const void* k_biases, const uint32_t* v_codes, const void* v_scales,
                    const void* v_biases, qlin_dtype sb_dtype, void* ws, int64_t ws_bytes, void* out,
                    qlin_dtype out_dtype, void* stream) {
  const bool own = ws == nullptr;
  if (!q || !k_codes || !k_scales || !k_biases || !v_codes || !v_scales || !v_biases || !out) return QLIN_ERR_NULL;
  if ((q_dtype != QLIN_F16 && q_dtype != QLIN_BF16) || (sb_dtype != QLIN_F16 && sb_dtype != QLIN_BF16) ||
      (out_dtype != QLIN_F32 && out_dtype != QLIN_F16 && out_dtype != QLIN_BF16))
    return QLIN_ERR_DTYPE;
  if (bits != 4 && bits != 8) return QLIN_ERR_BITS;
  if (heads < 1 || heads > 65536 || kv_heads < 1 || heads % kv_heads != 0 || n_rows < 1 || n_rows > (1 << 24))
    return QLIN_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512) return QLIN_ERR_SHAPE;
  if ((group_size != 32 && group_size != 64 && group_size != 128) || group_size > head_dim) return QLIN_ERR_SHAPE;
  if (!aligned(q, 2) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_scales, 2) ||
      !aligned(k_biases, 2) || !aligned(v_scales, 2) || !aligned(v_biases, 2) || (!own && !aligned(ws, 4)) ||
      !aligned(out, dtype_size(out_dtype)))
    return QLIN_ERR_ALIGN;
  const int64_t need = qlin_kvq_decode_workspace(heads, n_rows, head_dim);
  if (!own && need > ws_bytes) return QLIN_ERR_ARG;
  if (own && need > (int64_t)QLIN_KVQ_SCRATCH_BYTES) return QLIN_ERR_SCRATCH;
  const size_t ob = (size_t)heads * head_dim * dtype_size(out_dtype);
  const size_t rows = (size_t)kv_heads * n_rows;
  const size_t cb = rows * head_dim * bits / 8, sbb = rows * (head_dim / group_size) * 2;
  if (overlaps(out, ob, q, (size_t)heads * head_dim * 2) || (!own && overlaps(out, ob, ws, (size_t)need)) ||
      overlaps(out, ob, k_codes, cb) || overlaps(out, ob, v_codes, cb) || overlaps(out, ob, k_scales, sbb) ||
      overlaps(out, ob, k_biases, sbb) || overlaps(out, ob, v_scales, sbb) || overlaps(out, ob, v_biases, sbb))
    return QLIN_ERR_ARG;
  if (!own) {
    for (const void* in : {static_cast<const void*>(q), static_cast<const void*>(k_codes),
                           static_cast<const void*>(v_codes), k_scales, k_biases, v_scales, v_biases}) {
      const size_t len = in == q ? (size_t)heads * head_dim * 2 : (in == k_codes || in == v_codes) ? cb : sbb;
      if (overlaps(ws, (size_t)need, in, len)) return QLIN_ERR_ARG;
    }
  }
  float* part = static_cast<float*>(ws);
  if (own && qlin::kvq_scratch(&part) != hipSuccess) return QLIN_ERR_HIP;
  qlin::KvqParams a{};
  a.q = q; a.q_dtype = q_dtype; a.q_vec = aligned(q, 16) ? 1 : 0; a.kc = k_codes; a.ks = k_scales; a.kb = k_biases;
  a.vc = v_codes; a.vs = v_scales; a.vb = v_biases; a.sb_dtype = sb_dtype;
  a.H = heads; a.KV = kv_heads; a.N = n_rows; a.D = head_dim; a.GS = group_size; a.bits = bits;
  a.block = kvq_block(n_rows); a.G = (n_rows + a.block - 1) / a.block;
  a.opart = part;
  a.stats = a.opart + (size_t)heads * a.G * head_dim;
  a.out = out; a.out_dtype = out_dtype;
  if (qlin::launch_kvq_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess) return QLIN_ERR_HIP;
  g_dispatch[7].fetch_add(1, std::memory_order_relaxed);
  return QLIN_OK;
}
}  // namespace

qlin_status qlin_kvq_decode(const void* q, qlin_dtype q_dtype, int32_t heads, int32_t kv_heads, int32_t n_rows,
                            int32_t head_dim, int32_t group_size, int32_t bits, const uint32_t* k_codes,
                            const void* k_scales, const void* k_biases, const uint32_t* v_codes,
                            const void* v_scales, const void* v_biases, qlin_dtype sb_dtype, void* workspace,
                            int64_t workspace_bytes, void* out, qlin_dtype out_dtype, void* stream) {
  if (!workspace) return QLIN_ERR_NULL;
  return kvq_run(q, q_dtype, heads, kv_heads, n_rows, head_dim, group_size, bits, k_codes, k_scales, k_biases,
                 v_codes, v_scales, v_biases, sb_dtype, workspace, workspace_bytes, out, out_dtype, stream);
}

qlin_status qlin_kvq_decode_noalloc(const void* q, qlin_dtype q_dtype, int32_t heads, int32_t kv_heads,
                                    int32_t n_rows, int32_t head_dim, int32_t group_size, int32_t bits,
                                    const uint32_t* k_codes, const void* k_scales, const void* k_biases,
                                    const uint32_t* v_codes, const void* v_scales, const void* v_biases,
                                    qlin_dtype sb_dtype, void* out, qlin_dtype out_dtype, void* stream) {
  return kvq_run(q, q_dtype, heads, kv_heads, n_rows, head_dim, group_size, bits, k_codes, k_scales, k_biases,
                 v_codes, v_scales, v_biases, sb_dtype, nullptr, 0, out, out_dtype, stream);
}

int32_t qlin_set_path(int32_t path) {
  if (path < 0 || path > 2) return -1;
  return g_path.exchange(path, std::memory_order_relaxed);
}

int32_t qlin_set_merge_spin_limit(int32_t limit) {
  if (limit < 0) return -1;
  return g_merge_spin.exchange(limit, std::memory_order_relaxed);
}

int64_t qlin_merge_timeouts(int32_t reset) {
  if (reset != 0 && reset != 1) return -1;
  unsigned int* p = nullptr;
  if (merge_timeouts_ptr(&p) != hipSuccess) return -1;
  unsigned int v = 0;
  if (hipMemcpy(&v, p, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return -1;
  if (reset && hipMemset(p, 0, sizeof(v)) != hipSuccess) return -1;
  return (int64_t)v;
}

int64_t qlin_dispatch_count(int32_t which) {
  if (which < 0 || which > 9) return -1;
  return g_dispatch[which].load(std::memory_order_relaxed);
}

const char* qlin_status_string(qlin_status s) {
  switch (s) {
    case QLIN_OK: return "ok";
    case QLIN_ERR_NULL: return "a required pointer is NULL";
    case QLIN_ERR_SHAPE: return "shape out of range (0 <= T <= 32, K a positive multiple of 64, N >= 0)";
    case QLIN_ERR_DTYPE: return "unsupported or inconsistent dtype";
    case QLIN_ERR_BITS: return "bits must be 4, 8 or 16 and group_size 64";
    case QLIN_ERR_ALIGN: return "pointer misaligned";
    case QLIN_ERR_HIP: return "HIP runtime error";
    case QLIN_ERR_ARG: return "invalid argument";
    case QLIN_ERR_SCRATCH: return "the call needs more device scratch than the static buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
