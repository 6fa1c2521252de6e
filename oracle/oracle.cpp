// liboracle — the plain, slow CPU reference for the decode-time fused quantized linear.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path (libqlin, its Python
// binding) may link, load or call this file; only the tests, the smoke check and
// the benchmark's CPU-baseline leg do.  It shares no code, header, table or
// constant generator with the HIP path.
//
// Sources (the pages this follows):
//   [p1] maya-mac, src/maya_mac/mlx_kernels.py — "Custom Metal kernels for the depth
//        decoder": module docstring, the `_linear_kernel` docstring (LayerNorm folding
//        identity), the 8-bit affine load, the LN finalize and the epilogue, `linear()`.
//   [p2] @mlx-bun/inference 0.0.0-stage -> 1.0.0, kernels/trellis/mixed-gate-up.ts —
//        silu(gate(x)) * up(x) for a few rows sharing one read of x.
//   [p3] mlx-bun 0.0.10 -> 0.0.12, model/fused-decode-kernel.ts — the 4-bit packing
//        (element j of a word at bits 4j, low nibble first) and the scale-factored dequant.
//
// What it computes is the plain definition, not the fast method:
//   W[n,k]   = q[n,k] * s[n,k/64] + b[n,k/64]              (exact in fp64)
//   xhat     = two-pass LayerNorm of x in fp64 (biased variance, eps), or x itself
//   z[t,n]   = sum_k xhat[t,k] * W[n,k]                     (fp64, k ascending)
//   y        = [add +] [res +] act(z)      act = exact-erf GELU or none
//   gate/up  = silu(z_gate) * z_up
//   attend   = the band's cache with this pass's keys and values appended, and causal
//              softmax attention of the new positions over it (at most 32 positions)
//   sample   = exact top-k by the logits' order-preserving keys (ties with the k-th kept),
//              Gumbel-max over the kept codes, and the chosen code's embedding appended
//   kvq      = one query position's attention over an affine-quantized K/V cache
// Everything is computed in double precision from the exact bit patterns the GPU
// receives.  Build: g++ -O2 -std=c++17 -fPIC -shared -ffp-contract=off (no fast-math).
//
// Parity pins for every function live in tests/test_oracle_*.py.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <vector>
#include <limits>

namespace {

// ---------------------------------------------------------------------------
// 16-bit float formats, written out from their definitions.
//   binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
//   bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits (the top half of binary32).
// ---------------------------------------------------------------------------

double decode_fp(uint32_t bits, int exp_bits, int frac_bits) {
  const uint32_t sign = bits >> (exp_bits + frac_bits);
  const uint32_t e = (bits >> frac_bits) & ((1u << exp_bits) - 1u);
  const uint32_t f = bits & ((1u << frac_bits) - 1u);
  const int bias = (1 << (exp_bits - 1)) - 1;
  double v;
  if (e == (1u << exp_bits) - 1u) {
    v = f ? std::numeric_limits<double>::quiet_NaN() : std::numeric_limits<double>::infinity();
  } else if (e == 0) {
    v = std::ldexp((double)f, 1 - bias - frac_bits);                       // subnormal
  } else {
    v = std::ldexp((double)(f | (1u << frac_bits)), (int)e - bias - frac_bits);
  }
  return sign ? -v : v;
}

// Round a double to the nearest representable value of the format, ties to even,
// and return its bit pattern.  Overflow goes to infinity (IEEE round-to-nearest).
uint32_t encode_fp_rne(double v, int exp_bits, int frac_bits) {
  const uint32_t sign_bit = 1u << (exp_bits + frac_bits);
  const uint32_t exp_all = (1u << exp_bits) - 1u;
  if (std::isnan(v)) return (exp_all << frac_bits) | (1u << (frac_bits - 1));  // canonical quiet NaN
  const uint32_t sign = std::signbit(v) ? sign_bit : 0u;
  double a = std::fabs(v);
  if (std::isinf(a)) return sign | (exp_all << frac_bits);
  if (a == 0.0) return sign;
  const int bias = (1 << (exp_bits - 1)) - 1;
  const int emin = 1 - bias;                              // smallest normal exponent
  int e = std::ilogb(a);                                   // floor(log2 a)
  if (e < emin) e = emin;                                  // subnormal range shares emin's spacing
  const double ulp = std::ldexp(1.0, e - frac_bits);
  const double r = std::nearbyint(a / ulp);                // a/ulp is exact; nearbyint is RNE
  double rounded = r * ulp;
  // largest finite: (2 - 2^-frac) * 2^(exp_all - 1 - bias)
  const double maxfin = std::ldexp((double)((2u << frac_bits) - 1u), (int)exp_all - 1 - bias - frac_bits);
  if (rounded > maxfin) return sign | (exp_all << frac_bits);
  // encode the (now exactly representable) value
  int re = std::ilogb(rounded);
  if (re < emin) {                                         // subnormal (or rounded to min normal handled below)
    const uint32_t f = (uint32_t)std::ldexp(rounded, -(emin - frac_bits));
    return sign | f;
  }
  const uint32_t f = (uint32_t)(std::ldexp(rounded, frac_bits - re)) - (1u << frac_bits);
  return sign | ((uint32_t)(re + bias) << frac_bits) | f;
}

double f16_to_f64(uint16_t h) { return decode_fp(h, 5, 10); }
double bf16_to_f64(uint16_t h) { return decode_fp(h, 8, 7); }

// dtype codes shared with the Python wrapper: 0 = fp32, 1 = fp16, 2 = bf16
double elem_to_f64(const void* p, int dtype, int64_t i) {
  if (dtype == 0) return (double)((const float*)p)[i];
  const uint16_t h = ((const uint16_t*)p)[i];
  return dtype == 1 ? f16_to_f64(h) : bf16_to_f64(h);
}

// ---------------------------------------------------------------------------
// Affine group quantization format.
//   [p1] 8-bit load: a row's codes are packed four to a 32-bit word, code j of a
//        word at bits 8j; scale and bias for element (n, k) sit at index
//        (n*K + k) / 64, i.e. an (N, K/64) row-major table.
//   [p3] 4-bit: eight codes to a word, element j at bits 4j (low nibble first).
// ---------------------------------------------------------------------------

constexpr int64_t GROUP = 64;

uint32_t code_at(const uint32_t* words, int64_t K, int bits, int64_t n, int64_t k) {
  const int64_t per_word = 32 / bits;
  const int64_t words_per_row = K / per_word;
  const uint32_t w = words[n * words_per_row + k / per_word];
  const uint32_t shift = (uint32_t)(bits * (k % per_word));
  return (w >> shift) & ((1u << bits) - 1u);
}

}  // namespace

extern "C" {

// ---- scalar format helpers (exported for the pins) ----
double orc_f16_to_f64(uint16_t h) { return f16_to_f64(h); }
double orc_bf16_to_f64(uint16_t h) { return bf16_to_f64(h); }
uint16_t orc_f64_to_f16(double v) { return (uint16_t)encode_fp_rne(v, 5, 10); }
uint16_t orc_f64_to_bf16(double v) { return (uint16_t)encode_fp_rne(v, 8, 7); }

// Round n doubles to the storage dtype (1 = fp16, 2 = bf16) with ties to even.
void orc_round(const double* in, int64_t n, int dtype, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (uint16_t)(dtype == 1 ? encode_fp_rne(in[i], 5, 10) : encode_fp_rne(in[i], 8, 7));
}

// Integer codes q[n, k] of a packed (N, K*bits/32) word array.
void orc_codes(const uint32_t* words, int64_t N, int64_t K, int bits, uint8_t* q) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) q[n * K + k] = (uint8_t)code_at(words, K, bits, n, k);
}

// W[n, k] = q * s + b in double precision (exact: q has at most 8 bits and s, b are binary16).
void orc_dequant_f64(const uint32_t* words, const uint16_t* scales, const uint16_t* biases,
                     int64_t N, int64_t K, int bits, double* W) {
  const int64_t G = K / GROUP;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const double s = f16_to_f64(scales[n * G + k / GROUP]);
      const double b = f16_to_f64(biases[n * G + k / GROUP]);
      W[n * K + k] = (double)code_at(words, K, bits, n, k) * s + b;
    }
}

// The single-precision dequantized value fl32(q * s + b) with one rounding (a fused
// multiply-add), which is what the library's unpack entry point must reproduce bit for bit.
void orc_dequant_f32(const uint32_t* words, const uint16_t* scales, const uint16_t* biases,
                     int64_t N, int64_t K, int bits, float* W) {
  const int64_t G = K / GROUP;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const float s = (float)f16_to_f64(scales[n * G + k / GROUP]);
      const float b = (float)f16_to_f64(biases[n * G + k / GROUP]);
      W[n * K + k] = std::fma((float)code_at(words, K, bits, n, k), s, b);
    }
}

// Affine quantizer, per row n and group of 64 consecutive k (the pages do not print
// their quantizer; this is the reading fixed for the library's pack entry point):
//   lo = min, hi = max of the group (binary32)
//   s  = fp16_rne( fl32( fl32(hi - lo) / (2^bits - 1) ) )
//   b  = fp16_rne( lo )
//   q  = s == 0 ? 0 : clamp( rint( fl32( fl32(w - b) / s ) ), 0, 2^bits - 1 )   (rint: ties to even)
// A group holding a NaN or infinity, or whose s or b overflows binary16, is marked bad:
// its codes are 0, s = +0, b = the canonical binary16 NaN 0x7E00, and *flag is set to 1.
// Codes are packed little-endian, code j of a word at bits bits*j.
// Returns the number of bad groups.
int64_t orc_pack_affine(const float* w, int64_t N, int64_t K, int bits,
                        uint32_t* words, uint16_t* scales, uint16_t* biases, int* flag) {
  const int64_t G = K / GROUP;
  const int64_t per_word = 32 / bits;
  const int64_t words_per_row = K / per_word;
  const float qmax = (float)((1 << bits) - 1);
  int64_t bad_groups = 0;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t i = 0; i < words_per_row; ++i) words[n * words_per_row + i] = 0u;
    for (int64_t g = 0; g < G; ++g) {
      const float* v = w + n * K + g * GROUP;
      bool finite = true;
      float lo = v[0], hi = v[0];
      for (int64_t j = 0; j < GROUP; ++j) {
        if (!std::isfinite(v[j])) finite = false;
        if (v[j] < lo) lo = v[j];
        if (v[j] > hi) hi = v[j];
      }
      bool bad = !finite;
      uint16_t s16 = 0, b16 = 0;
      if (!bad) {
        volatile float range = hi - lo;            // volatile: keep each binary32 rounding explicit
        volatile float s32 = range / qmax;
        s16 = (uint16_t)encode_fp_rne((double)s32, 5, 10);
        b16 = (uint16_t)encode_fp_rne((double)lo, 5, 10);
        if (!std::isfinite(f16_to_f64(s16)) || !std::isfinite(f16_to_f64(b16))) bad = true;
      }
      if (bad) {
        ++bad_groups;
        scales[n * G + g] = 0x0000;
        biases[n * G + g] = 0x7E00;
        continue;
      }
      scales[n * G + g] = s16;
      biases[n * G + g] = b16;
      const float s = (float)f16_to_f64(s16);
      const float b = (float)f16_to_f64(b16);
      for (int64_t j = 0; j < GROUP; ++j) {
        uint32_t q = 0;
        if (s != 0.0f) {
          volatile float diff = v[j] - b;
          volatile float ratio = diff / s;
          float r = std::rint((float)ratio);
          if (r < 0.0f) r = 0.0f;
          if (r > qmax) r = qmax;
          q = (uint32_t)r;
        }
        const int64_t k = g * GROUP + j;
        words[n * words_per_row + k / per_word] |= q << (uint32_t)(bits * (k % per_word));
      }
    }
  }
  if (bad_groups && flag) *flag = 1;
  return bad_groups;
}

// Two-pass LayerNorm of the T rows of x (T, K) into xhat (T, K), fp64:
//   mu = sum_k x / K;  var = sum_k (x - mu)^2 / K  (biased);  xhat = (x - mu) / sqrt(var + eps) * g + b
// [p1] LN finalize: biased variance, eps added before the reciprocal square root.
void orc_layernorm(const double* x, int64_t T, int64_t K, const double* gamma, const double* beta,
                   double eps, double* xhat) {
  for (int64_t t = 0; t < T; ++t) {
    const double* r = x + t * K;
    double mu = 0.0;
    for (int64_t k = 0; k < K; ++k) mu += r[k];
    mu /= (double)K;
    double var = 0.0;
    for (int64_t k = 0; k < K; ++k) var += (r[k] - mu) * (r[k] - mu);
    var /= (double)K;
    const double rstd = 1.0 / std::sqrt(var + eps);
    for (int64_t k = 0; k < K; ++k) xhat[t * K + k] = (r[k] - mu) * rstd * gamma[k] + beta[k];
  }
}

// Exact GELU, v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)), written with erfc so that it
// keeps full relative accuracy for v << 0.  [p1] the exact-erf GELU of the epilogue.
double orc_gelu(double v) { return 0.5 * v * std::erfc(-v / std::sqrt(2.0)); }

// silu(g) = g * sigmoid(g) = g / (1 + e^-g).  [p2] the SwiGLU tail.
double orc_silu(double g) { return g / (1.0 + std::exp(-g)); }

// Dense or dequantized weight matrix W (N, K) in fp64.
static void weight_f64(int bits, const void* wdata, int w_dtype, const uint16_t* scales,
                       const uint16_t* biases, int64_t N, int64_t K, std::vector<double>& W) {
  W.assign((size_t)(N * K), 0.0);
  if (bits == 16) {
    for (int64_t i = 0; i < N * K; ++i) W[(size_t)i] = elem_to_f64(wdata, w_dtype, i);
  } else {
    orc_dequant_f64((const uint32_t*)wdata, scales, biases, N, K, bits, W.data());
  }
}

// The activation rows the contraction sees: LN(x) or x, fp64.
static void activations_f64(const void* x, int x_dtype, int64_t T, int64_t K, const void* gamma,
                            const void* beta, double eps, int has_ln, std::vector<double>& a) {
  std::vector<double> xd((size_t)(T * K));
  for (int64_t i = 0; i < T * K; ++i) xd[(size_t)i] = elem_to_f64(x, x_dtype, i);
  if (!has_ln) { a = xd; return; }
  std::vector<double> g((size_t)K), b((size_t)K);
  for (int64_t k = 0; k < K; ++k) { g[(size_t)k] = elem_to_f64(gamma, x_dtype, k); b[(size_t)k] = elem_to_f64(beta, x_dtype, k); }
  a.assign((size_t)(T * K), 0.0);
  orc_layernorm(xd.data(), T, K, g.data(), b.data(), eps, a.data());
}

// z[t, n] = sum_k a[t, k] * W[n, k], k ascending, fp64.
static void contract(const std::vector<double>& a, const std::vector<double>& W, int64_t T, int64_t K,
                     int64_t N, double* z) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < N; ++n) {
      double s = 0.0;
      const double* ar = a.data() + t * K;
      const double* wr = W.data() + n * K;
      for (int64_t k = 0; k < K; ++k) s += ar[k] * wr[k];
      z[t * N + n] = s;
    }
}

// y (T, N) fp64 = [add +] [res +] act( LN?(x) . W^T )
//   [p1] `linear` docstring and the epilogue: the activation first, then the residual
//   row res[t, n], then the per-column constant add[n].
// x, gamma, beta, res, add are arrays of dtype x_dtype (1 = fp16, 2 = bf16).
// bits 16: wdata is an (N, K) dense array of dtype w_dtype; bits 8/4: packed words.
// act: 0 none, 1 exact GELU.  Returns 0, or -1 on an argument the oracle does not handle.
int orc_linear(const void* x, int x_dtype, int64_t T, int64_t K, int64_t N,
               int bits, const void* wdata, int w_dtype, const uint16_t* scales, const uint16_t* biases,
               int has_ln, const void* gamma, const void* beta, double eps,
               int act, const void* res, const void* add, double* y) {
  if (T < 0 || N < 0 || K <= 0 || K % GROUP) return -1;
  if (bits != 4 && bits != 8 && bits != 16) return -1;
  std::vector<double> a, W;
  activations_f64(x, x_dtype, T, K, gamma, beta, eps, has_ln, a);
  weight_f64(bits, wdata, w_dtype, scales, biases, N, K, W);
  contract(a, W, T, K, N, y);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < N; ++n) {
      double v = y[t * N + n];
      if (act == 1) v = orc_gelu(v);
      if (res) v += elem_to_f64(res, x_dtype, t * N + n);
      if (add) v += elem_to_f64(add, x_dtype, n);
      y[t * N + n] = v;
    }
  return 0;
}

// y (T, N) fp64 = silu(LN?(x) . Wg^T) * (LN?(x) . Wu^T).  [p2] gate and up read the
// same activation rows; the two projections share format, K and N.
int orc_gateup(const void* x, int x_dtype, int64_t T, int64_t K, int64_t N, int bits,
               const void* gdata, const uint16_t* gscales, const uint16_t* gbiases,
               const void* udata, const uint16_t* uscales, const uint16_t* ubiases, int w_dtype,
               int has_ln, const void* gamma, const void* beta, double eps, double* y) {
  if (T < 0 || N < 0 || K <= 0 || K % GROUP) return -1;
  if (bits != 4 && bits != 8 && bits != 16) return -1;
  std::vector<double> a, Wg, Wu;
  activations_f64(x, x_dtype, T, K, gamma, beta, eps, has_ln, a);
  std::vector<double> zg((size_t)(T * N)), zu((size_t)(T * N));
  weight_f64(bits, gdata, w_dtype, gscales, gbiases, N, K, Wg);
  contract(a, Wg, T, K, N, zg.data());
  Wg.clear(); Wg.shrink_to_fit();
  weight_f64(bits, udata, w_dtype, uscales, ubiases, N, K, Wu);
  contract(a, Wu, T, K, N, zu.data());
  for (int64_t i = 0; i < T * N; ++i) y[i] = orc_silu(zg[(size_t)i]) * zu[(size_t)i];
  return 0;
}

// ---------------------------------------------------------------------------
// attend — [p1] `_ATTEND` and `attend()`: one pass of a decoder layer's attention over a
// short band of positions.  It appends this pass's keys and values to the band's cache
// and runs causal softmax attention over at most 32 positions.
//   qkv (T, 3D), D = H * HD: per new position t, the query in columns [0, D), the key in
//       [D, 2D) and the value in [2D, 3D); head h owns columns h*HD .. h*HD + HD - 1 of each.
//   kv (2, H, P, HD): cached keys (index 0) and values (index 1) of P earlier positions.
//   kv_out (2, H, P + T, HD): the cache, then this pass's T rows (bit patterns copied).
//   For new position t (absolute position P + t) and head h, over keys j = 0 .. P + t
//   (the later positions are not visible: causal):
//       s_j = (q . k_j) / sqrt(HD)
//       p_j = exp(s_j - max_i s_i) / sum_i exp(s_i - max_i s_i)
//       out[t, h*HD + d] = sum_j p_j * v_j[d]
//   last = 1 asks for the last new position's row only (out has one row).
// Everything in fp64 from the exact input values; out is fp64, kv_out the copied bits.
// Returns 0, or -1 on an argument the oracle does not handle.
// ---------------------------------------------------------------------------
int orc_attend(const uint16_t* qkv, const uint16_t* kv, int dtype, int64_t P, int64_t T, int64_t H,
               int64_t HD, int last, double* out, uint16_t* kv_out) {
  if (P < 0 || T < 1 || H < 1 || HD < 1 || P + T > 32) return -1;
  if (P > 0 && !kv) return -1;
  const int64_t D = H * HD, L = P + T;
  // the cache, then the new rows
  for (int64_t i = 0; i < 2; ++i)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t j = 0; j < L; ++j)
        for (int64_t d = 0; d < HD; ++d) {
          const uint16_t v = j < P ? kv[((i * H + h) * P + j) * HD + d]
                                   : qkv[(j - P) * 3 * D + (1 + i) * D + h * HD + d];
          kv_out[((i * H + h) * L + j) * HD + d] = v;
        }
  auto val = [&](uint16_t b) { return dtype == 1 ? f16_to_f64(b) : bf16_to_f64(b); };
  // key or value row of absolute position j, head h, dimension d (i = 0 key, 1 value)
  auto kvv = [&](int64_t i, int64_t h, int64_t j, int64_t d) { return val(kv_out[((i * H + h) * L + j) * HD + d]); };
  const double scale = 1.0 / std::sqrt((double)HD);
  std::vector<double> s((size_t)L), pr((size_t)L);
  for (int64_t t = last ? T - 1 : 0; t < T; ++t) {
    const int64_t row = last ? 0 : t, pos = P + t;
    for (int64_t h = 0; h < H; ++h) {
      double m = -std::numeric_limits<double>::infinity();
      for (int64_t j = 0; j <= pos; ++j) {
        double a = 0.0;
        for (int64_t d = 0; d < HD; ++d) a += val(qkv[t * 3 * D + h * HD + d]) * kvv(0, h, j, d);
        s[(size_t)j] = a * scale;
        if (s[(size_t)j] > m) m = s[(size_t)j];
      }
      double z = 0.0;
      for (int64_t j = 0; j <= pos; ++j) { pr[(size_t)j] = std::exp(s[(size_t)j] - m); z += pr[(size_t)j]; }
      for (int64_t d = 0; d < HD; ++d) {
        double o = 0.0;
        for (int64_t j = 0; j <= pos; ++j) o += pr[(size_t)j] / z * kvv(1, h, j, d);
        out[row * D + h * HD + d] = o;
      }
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// sample — [p1] `_SAMPLE` and `sample()`: one sampling step of the depth decoder.
//   key(f)   = the order-preserving 32-bit key of the fp32 value f: bits u of f, ~u when the
//              sign bit is set, u | 2^31 otherwise (larger floats have larger keys; -0 < +0)
//   kth      = the top_k-th largest key over the n codes (sorting, not a radix select)
//   kept     = codes whose key >= kth (every code tied with the k-th is kept)
//   s_i      = fl32(fl32(f_i * inv_temp) + gumbel_i)   (two fp32 roundings, no fused
//              multiply-add: the argmax is an integer that fp32 rounding decides, so the
//              library computes it in the same precision)
//   code     = the kept i with the largest s_i, the smallest such i on ties; a NaN score
//              never wins; -1 when no kept score is a number
//   out      = prefix rows (n_prev, D) then, with a table, table row `code` (zeros when the
//              code is -1): element bit patterns copied, es bytes each
// logits: n values of dtype (0 fp32, 1 fp16, 2 bf16).  kept_count receives |kept|.
// ---------------------------------------------------------------------------
int orc_sample(const void* logits, int dtype, int64_t n, const float* gumbel, float inv_temp, int64_t top_k,
               const void* table, const void* prefix, int64_t n_prev, int64_t D, int64_t es, void* out,
               int32_t* code, int64_t* kept_count) {
  if (n < 1 || top_k < 1 || top_k > n || (es != 2 && es != 4) || D < 0 || n_prev < 0) return -1;
  std::vector<float> f((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    if (dtype == 0) f[(size_t)i] = static_cast<const float*>(logits)[i];
    else {
      const uint16_t b = static_cast<const uint16_t*>(logits)[i];
      f[(size_t)i] = (float)(dtype == 1 ? f16_to_f64(b) : bf16_to_f64(b));   // exact widening
    }
  }
  auto key = [](float v) {
    uint32_t u;
    std::memcpy(&u, &v, 4);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  };
  std::vector<uint32_t> keys((size_t)n);
  for (int64_t i = 0; i < n; ++i) keys[(size_t)i] = key(f[(size_t)i]);
  std::vector<uint32_t> sorted = keys;
  std::sort(sorted.begin(), sorted.end(), std::greater<uint32_t>());
  const uint32_t kth = sorted[(size_t)(top_k - 1)];
  int64_t best = -1, kept = 0;
  float bs = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    if (keys[(size_t)i] < kth) continue;
    ++kept;
    const float scaled = f[(size_t)i] * inv_temp;   // rounded to fp32
    const float sc = scaled + gumbel[i];             // rounded to fp32
    if (std::isnan(sc)) continue;
    if (best < 0 || sc > bs) { best = i; bs = sc; }   // ascending i: equal scores keep the smaller i
  }
  *code = (int32_t)best;
  *kept_count = kept;
  unsigned char* o = static_cast<unsigned char*>(out);
  const size_t row = (size_t)D * (size_t)es;
  if (n_prev > 0) std::memcpy(o, prefix, (size_t)n_prev * row);
  if (table) {
    if (best >= 0) std::memcpy(o + (size_t)n_prev * row, static_cast<const unsigned char*>(table) + (size_t)best * row, row);
    else std::memset(o + (size_t)n_prev * row, 0, row);
  }
  return 0;
}

// ---------------------------------------------------------------------------
// kvq decode — [p3] mlx-bun 0.0.10 -> 0.0.12, model/fused-decode-kernel.ts: attention of one
// query position over a quantized K/V cache (the kernel's own split into blocks and merge
// is a schedule; this is the plain definition it computes).
//   K[c, n, d] = qk * sk[c, n, d / GS] + bk[c, n, d / GS]      (affine, exact in fp64)
//   V[c, n, d] likewise
//   s[h, n]    = sum_d q[h, d] K[c, n, d]          c = h / (H / KV)  (query heads share KV heads)
//   out[h, d]  = sum_n softmax_n(s[h, .]) V[c, n, d]
// q arrives already scaled (the page's kernel applies no 1/sqrt(D)).  Codes: element d of
// a row at word d / (32 / bits), bits (d mod (32 / bits)) * bits, low bits first.
// q: (H, D) bit patterns of q_dtype; scales/biases bit patterns of sb_dtype (1 fp16, 2 bf16).
// ---------------------------------------------------------------------------
int orc_kvq_decode(const uint16_t* q, int q_dtype, const uint32_t* kc, const uint16_t* ks, const uint16_t* kb,
                   const uint32_t* vc, const uint16_t* vs, const uint16_t* vb, int sb_dtype, int64_t H, int64_t KV,
                   int64_t N, int64_t D, int64_t GS, int bits, double* out) {
  if (H < 1 || KV < 1 || H % KV != 0 || N < 1 || D < 1 || GS < 1 || D % GS != 0 || (bits != 4 && bits != 8) ||
      D % (32 / bits) != 0)
    return -1;
  auto val = [](uint16_t b, int dt) { return dt == 1 ? f16_to_f64(b) : bf16_to_f64(b); };
  const int64_t per = 32 / bits, words = D / per, groups = D / GS, rep = H / KV;
  const uint32_t mask = (1u << bits) - 1u;
  auto deq = [&](const uint32_t* c, const uint16_t* s, const uint16_t* b, int64_t kvh, int64_t n, int64_t d) {
    const int64_t row = kvh * N + n;
    const uint32_t code = (c[row * words + d / per] >> ((d % per) * bits)) & mask;
    return (double)code * val(s[row * groups + d / GS], sb_dtype) + val(b[row * groups + d / GS], sb_dtype);
  };
  std::vector<double> sc((size_t)N);
  for (int64_t h = 0; h < H; ++h) {
    const int64_t c = h / rep;
    double m = -std::numeric_limits<double>::infinity();
    for (int64_t n = 0; n < N; ++n) {
      double a = 0.0;
      for (int64_t d = 0; d < D; ++d) a += val(q[h * D + d], q_dtype) * deq(kc, ks, kb, c, n, d);
      sc[(size_t)n] = a;
      if (a > m) m = a;
    }
    double z = 0.0;
    for (int64_t n = 0; n < N; ++n) { sc[(size_t)n] = std::exp(sc[(size_t)n] - m); z += sc[(size_t)n]; }
    for (int64_t d = 0; d < D; ++d) {
      double o = 0.0;
      for (int64_t n = 0; n < N; ++n) o += sc[(size_t)n] / z * deq(vc, vs, vb, c, n, d);
      out[h * D + d] = o;
    }
  }
  return 0;
}

}  // extern "C"
