/*
 * qlin.h — C ABI of libqlin, the MI355X (gfx950) decode-time fused quantized linear.
 *
 * The operation ([p1] maya-mac src/maya_mac/mlx_kernels.py, module docstring and the
 * `linear` docstring):
 *
 *     y = [add +] [res +] act( LN?(x) . dequant(W)^T )          x: (T, K), W: (N, K), y: (T, N)
 *
 * for a few activation rows (1 <= T <= 32) against either a dense fp16/bf16 W or affine
 * group-quantized codes: 8-bit or 4-bit unsigned codes q with one fp16 scale s and one
 * fp16 bias b per group of 64 consecutive k, W[n, k] = q * s[n, k/64] + b[n, k/64]
 * ([p1] the 8-bit load of `_linear_kernel`; [p3] mlx-bun 0.0.10 -> 0.0.12,
 * model/fused-decode-kernel.ts for the 4-bit layout).  The optional LayerNorm prologue
 * (biased variance, eps inside the square root) is folded into the weight stream with the
 * single-pass shifted statistics ([p1] `_linear_kernel` docstring).  The epilogue applies,
 * in this order, exact-erf GELU, the residual row and the per-column constant ([p1] the
 * epilogue of `_linear_kernel`).  qlin_gateup_swiglu computes silu(x.Wg^T) * (x.Wu^T) over
 * one read of x ([p2] @mlx-bun/inference 0.0.0-stage -> 1.0.0, kernels/trellis/
 * mixed-gate-up.ts).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc or a torch CUDA tensor's
 *     data_ptr) unless stated otherwise; all arrays are dense and row-major.
 *   - The caller allocates and owns every buffer; inputs are only read (borrowed).
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.  Calls only
 *     enqueue work on it and return: no allocation, no synchronization, no device query
 *     after the first call on a device, so they may be recorded into a hipGraph.
 *   - Arguments are validated on the host before any HIP call.  On any error the function
 *     returns a negative qlin_status, enqueues nothing and leaves every output untouched.
 *     Nothing is thrown across the ABI.
 *   - Results are deterministic: the same inputs give bitwise-identical outputs (no
 *     floating-point atomics; every cross-lane and cross-wave sum has a fixed order).
 */
#ifndef QLIN_H
#define QLIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes, dtype codes and activation codes travel as plain 32-bit integers: a caller
 * may pass any value, and an out-of-range one is rejected with a status (an enum parameter
 * type would make such a value undefined behaviour in C++ before it could be checked). */
typedef int32_t qlin_status;
enum {
  QLIN_OK = 0,
  QLIN_ERR_NULL = -1,   /* a required pointer is NULL */
  QLIN_ERR_SHAPE = -2,  /* T, K or N outside the accepted range */
  QLIN_ERR_DTYPE = -3,  /* unsupported or inconsistent dtype */
  QLIN_ERR_BITS = -4,   /* bits not in {4, 8, 16} or group_size != 64 */
  QLIN_ERR_ALIGN = -5,  /* a pointer does not have the required alignment */
  QLIN_ERR_HIP = -6,    /* the HIP runtime reported an error */
  QLIN_ERR_ARG = -7,    /* any other invalid argument (act code, eps, n_passes, ...) */
  QLIN_ERR_SCRATCH = -8 /* the call needs more than the library's static device scratch */
};

typedef int32_t qlin_dtype;
enum { QLIN_F32 = 0, QLIN_F16 = 1, QLIN_BF16 = 2 };

typedef int32_t qlin_act;
enum { QLIN_ACT_NONE = 0, QLIN_ACT_GELU = 1 };

/* A weight matrix W of N output rows and K input columns (y = x . W^T).
 *   bits == 16: dense; `data` holds N*K elements of `dtype` (QLIN_F16 or QLIN_BF16, and it
 *               must equal the activation dtype); scales and biases are ignored (may be NULL).
 *   bits == 8 or 4: `data` holds N rows of K*bits/32 uint32 words; within a row, code k sits
 *               in word k/(32/bits) at bits bits*(k mod (32/bits)) (low bits first).
 *               `scales` and `biases` hold N rows of K/64 fp16 values; `dtype` must be
 *               QLIN_F16 (the scale/bias dtype).
 * group_size must be 64.  K must be a positive multiple of 64.
 * Alignment: data 16 bytes; scales and biases 2 bytes. */
typedef struct {
  int32_t bits;
  int32_t group_size;
  int64_t N;
  int64_t K;
  int32_t dtype;
  const void* data;
  const void* scales;
  const void* biases;
} qlin_weight;

/* LayerNorm prologue parameters: gamma and beta hold K elements of the activation dtype
 * (16-byte aligned); eps > 0 is added to the biased variance before the square root
 * (eps == 0 is accepted too). */
typedef struct {
  const void* gamma;
  const void* beta;
  float eps;
} qlin_ln;

/* y = [add +] [res +] act( LN?(x) . dequant(w)^T )
 *   x         (T, K) of x_dtype (QLIN_F16 or QLIN_BF16), 16-byte aligned.
 *   T         number of activation rows, 0 <= T <= 32 (T == 0 is a no-op).
 *   w         the weight, w->N >= 0 (N == 0 is a no-op), w->K == the row length of x.
 *   ln        NULL for no LayerNorm, else the prologue parameters.
 *   act       QLIN_ACT_NONE or QLIN_ACT_GELU (0.5 v (1 + erf(v / sqrt 2))).
 *   residual  NULL or (T, N) of x_dtype, added after the activation.
 *   add       NULL or (N,) of x_dtype, added last.
 *   y         (T, N) of y_dtype (QLIN_F32, QLIN_F16 or QLIN_BF16), written with one
 *             round-to-nearest-even from an fp32 value; it must not overlap x or residual.
 *   stream    hipStream_t as void*.
 * Accumulation is fp32.  Each activation enters the contraction with an error of at most
 * 2^-22 times the largest magnitude among the elements of its row in the same aligned
 * block of 512 (with LayerNorm, of the values (x - x[t, 0]) * gamma).  Returns QLIN_OK once
 * the work is enqueued. */
qlin_status qlin_linear(const void* x, qlin_dtype x_dtype, int32_t T, const qlin_weight* w,
                        const qlin_ln* ln, qlin_act act, const void* residual, const void* add,
                        void* y, qlin_dtype y_dtype, void* stream);

/* y = silu(LN?(x) . gate^T) * (LN?(x) . up^T), silu(g) = g / (1 + e^-g), computed in fp32
 * and rounded once to y_dtype.  gate and up must have the same bits, group size, N, K and
 * dtype.  Other arguments as in qlin_linear; y is (T, N). */
qlin_status qlin_gateup_swiglu(const void* x, qlin_dtype x_dtype, int32_t T, const qlin_weight* gate,
                               const qlin_weight* up, const qlin_ln* ln, void* y, qlin_dtype y_dtype,
                               void* stream);

/* The MLP of a decoder layer, gate+up then down ([p3] mlx-bun 0.0.10 -> 0.0.12,
 * model/fused-mlp-kernel.ts, whose header comment states the whole-MLP product):
 *     h = silu(LN?(x) . gate^T) * (LN?(x) . up^T)    (T, I), rounded once to x_dtype
 *     y = [residual +] h . down^T                     (T, Hout), rounded once to y_dtype
 * as two dispatches on `stream`: the gate/up kernel writes h, then the fused linear reads
 * it with the residual in its epilogue.  The page's single dispatch adds the down partials
 * with floating-point atomics; here no atomic touches data, so y is bitwise reproducible.
 * The hidden activation is rounded to the activation dtype, as the page rounds it to bf16.
 *   gate, up   (I, K) weights as for qlin_gateup_swiglu;  down (Hout, I): down->K == I.
 *   h          caller-owned device workspace of T*I elements of x_dtype, 16-byte aligned;
 *              it must not overlap x, the weights, residual or y.  On return its contents
 *              are h (the call may be captured: h is written when the work runs).
 *   residual   (T, Hout) of x_dtype or NULL;  y (T, Hout) of y_dtype, not overlapping x,
 *              h or residual.
 * Both stages are validated before anything is enqueued; errors as for qlin_linear. */
qlin_status qlin_mlp(const void* x, qlin_dtype x_dtype, int32_t T, const qlin_weight* gate,
                     const qlin_weight* up, const qlin_weight* down, const qlin_ln* ln,
                     const void* residual, void* h, void* y, qlin_dtype y_dtype, void* stream);

/* Quantize an fp32 (N, K) matrix w (device, 16-byte aligned) to the affine format above.
 * For each row n and group of 64 consecutive k, in IEEE binary32 with ties to even:
 *     lo = min, hi = max;  s = fp16(fl32(fl32(hi - lo) / (2^bits - 1)));  b = fp16(lo);
 *     q = s == 0 ? 0 : clamp(rint(fl32(fl32(w - b) / s)), 0, 2^bits - 1)
 * (the pages do not print their quantizer; this is the library's definition).  A group
 * that holds a NaN or infinity, or whose s or b overflows fp16, is written as q = 0,
 * s = +0, b = fp16 NaN (0x7E00), and *nonfinite_flag (a device int, may be NULL) is set
 * to 1; the flag is never cleared by this call.
 *   codes   (N, K*bits/32) uint32, 16-byte aligned;  scales, biases (N, K/64) of sb_dtype.
 *   bits    4 or 8;  group_size 64;  sb_dtype QLIN_F16. */
qlin_status qlin_pack_affine(const float* w, int64_t N, int64_t K, int32_t bits, int32_t group_size,
                             uint32_t* codes, void* scales, void* biases, qlin_dtype sb_dtype,
                             int32_t* nonfinite_flag, void* stream);

/* Dequantize w into out (N, K) fp32 (device): out = fmaf(q, s, b) with one rounding for
 * quantized weights, or the widened element for dense ones.  Test and diagnostic use. */
qlin_status qlin_unpack_affine(const qlin_weight* w, float* out, void* stream);

/* Validation only: returns what qlin_linear / qlin_gateup_swiglu would return for these
 * arguments without enqueueing anything (the "is this call servable" predicate).  `up`
 * is NULL for a plain linear.  Needs no GPU. */
qlin_status qlin_check(const void* x, qlin_dtype x_dtype, int32_t T, const qlin_weight* w,
                       const qlin_weight* up, const qlin_ln* ln, qlin_act act, const void* residual,
                       const void* add, const void* y, qlin_dtype y_dtype);

/* One pass of a chain of dependent fused linears ([p1] module docstring: the depth decoder
 * runs 124 small dependent layer passes per frame).  Fields as in qlin_linear; ln_gamma
 * NULL means no LayerNorm. */
typedef struct {
  const void* x;
  int32_t T;
  qlin_weight w;
  const void* ln_gamma;
  const void* ln_beta;
  float ln_eps;
  int32_t act;
  const void* residual;
  const void* add;
  void* y;
} qlin_pass;

typedef struct qlin_chain qlin_chain;

/* Record n_passes (>= 1) fused linears, in order, into one hipGraph by stream capture on
 * `capture_stream` (which must not be capturing already) and instantiate it.  Every pass
 * is validated first; on error nothing is recorded and *out is NULL.  The pass array is
 * copied; the device buffers it names must stay valid while the chain is used.  Allocates
 * host and graph memory (a setup call, not capture-safe itself).  Returns QLIN_ERR_HIP if
 * capture or instantiation fails. */
qlin_status qlin_chain_create(const qlin_pass* passes, int32_t n_passes, qlin_dtype x_dtype,
                              qlin_dtype y_dtype, void* capture_stream, qlin_chain** out);

/* Launch the recorded chain once on `stream` (asynchronous). */
qlin_status qlin_chain_launch(qlin_chain* chain, void* stream);

/* Number of passes recorded in `chain` (0 for NULL). */
int32_t qlin_chain_passes(const qlin_chain* chain);

/* Release the graph and its host memory.  NULL is ignored. */
void qlin_chain_destroy(qlin_chain* chain);

/* Attention of one decoder-layer pass over a short band of positions ([p1] maya-mac
 * src/maya_mac/mlx_kernels.py, `_ATTEND` and `attend()`): append this pass's keys and
 * values to the band's cache, then causal softmax attention of the new positions.
 *   qkv      (T, 3D) of dtype (QLIN_F16 or QLIN_BF16), D = heads * head_dim: per new
 *            position the query (columns [0, D)), key ([D, 2D)) and value ([2D, 3D)) of
 *            every head; head h owns head_dim consecutive columns of each.  16-byte aligned.
 *   kv       (2, heads, P, head_dim) of dtype: the cached keys (index 0) and values (1) of
 *            the P earlier positions; may be NULL when P == 0.  16-byte aligned.
 *   P, T     0 <= P, 1 <= T, P + T <= 32.
 *   heads    1 .. 65536;  head_dim a multiple of 16 in [16, 512].
 *   last     0: out is (T, D), one row per new position;  1: out is (1, D), the last new
 *            position's row only.
 *   out      of out_dtype (QLIN_F32, QLIN_F16 or QLIN_BF16): row t, columns h*head_dim + d
 *            hold sum_{j <= P + t} p_j v_j[d], p = softmax over j of (q_t . k_j) / sqrt(head_dim)
 *            (position P + t sees keys 0 .. P + t only), computed in fp32 and rounded once.
 *   kv_out   (2, heads, P + T, head_dim) of dtype: the cache, then this pass's T rows (bit
 *            patterns copied).  It must not overlap qkv or kv; out must not overlap any input
 *            or kv_out.
 * Returns QLIN_OK once the work is enqueued; argument errors as for qlin_linear. */
qlin_status qlin_attend(const void* qkv, const void* kv, qlin_dtype dtype, int32_t P, int32_t T, int32_t heads,
                        int32_t head_dim, int32_t last, void* out, qlin_dtype out_dtype, void* kv_out, void* stream);

/* Validation only: what qlin_attend would return for these arguments, with nothing
 * enqueued.  Needs no GPU. */
qlin_status qlin_attend_check(const void* qkv, const void* kv, qlin_dtype dtype, int32_t P, int32_t T,
                              int32_t heads, int32_t head_dim, int32_t last, const void* out, qlin_dtype out_dtype,
                              const void* kv_out);

/* One sampling step of the depth decoder ([p1] maya-mac src/maya_mac/mlx_kernels.py,
 * `_SAMPLE` and `sample()`): exact top-k of the logits, Gumbel-max over the kept codes, and
 * the chosen code's embedding appended to the prefix.
 *   logits     (n) of logit_dtype (QLIN_F32, QLIN_F16 or QLIN_BF16), 1 <= n <= 8192,
 *              aligned to its element size.  Each logit f (widened exactly to fp32) has the
 *              order-preserving key of its bits u: ~u when the sign bit is set, u | 2^31
 *              otherwise (larger floats have larger keys; -0 orders below +0).
 *   top_k      1 <= top_k <= n: codes whose key is >= the top_k-th largest key are kept
 *              (all codes tied with the k-th value are kept).
 *   gumbel     (n) fp32 noise of this step (the caller draws it, e.g. one row per level).
 *   inv_temp   finite and > 0.  The score of a kept code is fl32(fl32(f * inv_temp) + g),
 *              two fp32 roundings (no fused multiply-add).
 *   code       device int32: the kept code with the largest score, the smallest index among
 *              equal scores; a NaN score never wins; -1 if no kept score is a number.
 *   table      (n, D) of emb_dtype: this step's code embeddings, or NULL (nothing appended).
 *   prefix     (n_prev, D) of emb_dtype, or NULL when n_prev == 0.
 *   out        (n_prev + (table != NULL), D) of emb_dtype: the prefix rows, then table row
 *              `code` (zeros when code is -1), bit patterns copied.  out may be the prefix
 *              itself (then only the new row is written); otherwise it must not overlap it.
 *   D          row width; D * sizeof(emb_dtype) a multiple of 16; table, prefix and out
 *              16-byte aligned.
 * Errors: QLIN_ERR_NULL, QLIN_ERR_SHAPE (n, top_k, D, n_prev), QLIN_ERR_DTYPE,
 * QLIN_ERR_ALIGN, QLIN_ERR_ARG (inv_temp, overlaps) before any HIP call. */
qlin_status qlin_sample(const void* logits, qlin_dtype logit_dtype, int32_t n, const float* gumbel, float inv_temp,
                        int32_t top_k, const void* table, const void* prefix, int32_t n_prev, int32_t D,
                        qlin_dtype emb_dtype, void* out, int32_t* code, void* stream);

/* Attention of one query position per head over an affine-quantized K/V cache ([p3]
 * mlx-bun 0.0.10 -> 0.0.12, model/fused-decode-kernel.ts, flash decoding split over rows):
 *     s[h, n]   = sum_d q[h, d] K[c, n, d],    c = h / (heads / kv_heads)
 *     out[h, d] = sum_n softmax_n(s[h, .]) V[c, n, d]
 * with K (and V) = code * scale + bias per group of group_size elements along d (the weight
 * format above, rows of head_dim elements).  q arrives already scaled (no 1/sqrt(head_dim)
 * is applied).  Computed in fp32 (online softmax per block of rows, then a merge of the
 * blocks in order) and rounded once to out_dtype.  Two dispatches; no atomics.
 *   q          (heads, head_dim) of q_dtype (QLIN_F16 or QLIN_BF16), 2-byte aligned.
 *   heads      1..65536, a multiple of kv_heads;  n_rows 1..2^24;  head_dim 64, 128, 256 or
 *              512;  group_size 32, 64 or 128 (<= head_dim);  bits 4 or 8.
 *   k_codes    (kv_heads, n_rows, head_dim*bits/32) uint32, 16-byte aligned; k_scales,
 *              k_biases (kv_heads, n_rows, head_dim/group_size) of sb_dtype (QLIN_F16 or
 *              QLIN_BF16); v_* likewise.
 *   workspace  device scratch of at least qlin_kvq_decode_workspace(heads, n_rows, head_dim)
 *              bytes, 4-byte aligned, owned by the caller (partials of the row blocks).
 *   out        (heads, head_dim) of out_dtype (QLIN_F32, QLIN_F16 or QLIN_BF16); it must not
 *              overlap the inputs or the workspace.
 * Errors as for qlin_linear, before any HIP call (QLIN_ERR_ARG for a small workspace). */
int64_t qlin_kvq_decode_workspace(int32_t heads, int32_t n_rows, int32_t head_dim);
qlin_status qlin_kvq_decode(const void* q, qlin_dtype q_dtype, int32_t heads, int32_t kv_heads, int32_t n_rows,
                            int32_t head_dim, int32_t group_size, int32_t bits, const uint32_t* k_codes,
                            const void* k_scales, const void* k_biases, const uint32_t* v_codes,
                            const void* v_scales, const void* v_biases, qlin_dtype sb_dtype, void* workspace,
                            int64_t workspace_bytes, void* out, qlin_dtype out_dtype, void* stream);

/* qlin_kvq_decode without the workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The block partials go to a static device array of QLIN_KVQ_SCRATCH_BYTES bytes that the
 * library holds on every GPU it runs on until the process ends; the call itself allocates
 * nothing.  Every call on one GPU shares that GPU's array: calls that may overlap in time
 * on one GPU (on different streams, or from several host threads) race and must be
 * serialized by the caller.  Nothing in the array needs to start at zero: each call writes
 * every partial it reads.  Arguments, layouts and errors as for qlin_kvq_decode, except
 * QLIN_ERR_SCRATCH (nothing enqueued) when qlin_kvq_decode_workspace(heads, n_rows,
 * head_dim) exceeds QLIN_KVQ_SCRATCH_BYTES, and QLIN_ERR_HIP when the array's device
 * address cannot be obtained on the current device (looked up on the first call there). */
#define QLIN_KVQ_SCRATCH_BYTES (8 << 20)
qlin_status qlin_kvq_decode_noalloc(const void* q, qlin_dtype q_dtype, int32_t heads, int32_t kv_heads,
                                    int32_t n_rows, int32_t head_dim, int32_t group_size, int32_t bits,
                                    const uint32_t* k_codes, const void* k_scales, const void* k_biases,
                                    const uint32_t* v_codes, const void* v_scales, const void* v_biases,
                                    qlin_dtype sb_dtype, void* out, qlin_dtype out_dtype, void* stream);

/* ---- measurement aid ----------------------------------------------------------------
 * qlin_stream_read: the device's streaming-read ceiling for the weight stream's access (the
 * "HBM bandwidth" the pages' 8-bit-versus-fp16 timing comparison of the maya-mac depth
 * decoder kernels turns on, section "Custom Metal kernels for the depth decoder"): one
 * plain pass of 16-byte loads over a buffer, no other work.  Timing it over the same bytes
 * as a fused call gives the rate a pure read reaches on this device.
 *   buf      device pointer, 16-byte aligned; bytes a positive multiple of 16.  Read only.
 *   partial  device array of QLIN_STREAM_READ_BLOCKS uint32 (4-byte aligned), owned by the
 *            caller: block b of the launch writes the XOR of the 32-bit words it read to
 *            partial[b]; blocks past min(compute units, QLIN_STREAM_READ_BLOCKS) write
 *            nothing.  The XOR of all written entries is the XOR of every word of buf.
 * Errors: QLIN_ERR_NULL, QLIN_ERR_SHAPE, QLIN_ERR_ALIGN before any HIP call; QLIN_ERR_HIP
 * on a launch failure. */
#define QLIN_STREAM_READ_BLOCKS 1024
qlin_status qlin_stream_read(const void* buf, int64_t bytes, uint32_t* partial, void* stream);

/* The same read with its launch chosen by the caller, so that a measurement can take the best
 * of several: `blocks` workgroups of 512 threads (1 .. QLIN_STREAM_READ_BLOCKS; blocks past
 * it write nothing), `unroll` 16-byte loads in flight per thread (1, 2, 4, 8 or 16), and
 * non-temporal loads when `nontemporal` is 1 (0: ordinary loads).  qlin_stream_read is
 * blocks = min(compute units, QLIN_STREAM_READ_BLOCKS), unroll 4, non-temporal.
 * Errors as qlin_stream_read, plus QLIN_ERR_ARG for an unsupported launch. */
qlin_status qlin_stream_read_config(const void* buf, int64_t bytes, uint32_t* partial, int32_t blocks,
                                    int32_t unroll, int32_t nontemporal, void* stream);

/* Number of kernels this library has enqueued in this process, by entry point:
 * 0 = linear, 1 = gate/up, 2 = pack, 3 = unpack, 4 = attend, 5 = stream read, 6 = sample,
 * 7 = quantized-KV decode (a test can assert a kernel ran; qlin_mlp counts one gate/up and
 * one linear); 8 = how many of the linear and gate/up launches ran on the int8 streaming
 * kernel, 9 = how many on the vector-ALU kernel (the rest ran on the general kernel).  -1
 * for any other index. */
int64_t qlin_dispatch_count(int32_t which);

/* Selects the kernel family for 4- and 8-bit qlin_linear / qlin_gateup_swiglu / qlin_mlp
 * calls made after it, process-wide: 0 (the default) lets the library pick the int8 streaming
 * kernel wherever its shape rules admit the call and the general kernel elsewhere; 1 sends
 * every call to the general kernel; 2 sends calls of at most 4 activation rows to the
 * vector-ALU kernel where its shape rules admit them (4- and 8-bit codes, or dense fp16
 * weights with fp16 activations; K up to 4096, or 2048 with LayerNorm and 3-4 rows; no
 * LayerNorm with gate/up), the rest as 0.  All compute the same operation to
 * the same tolerance; this exists so that tests and measurements can exercise each one.
 * Returns the previous setting, or -1 (and changes nothing) for any other value.  Not
 * synchronized with calls in flight on other host threads. */
int32_t qlin_set_path(int32_t path);

/* The general kernel (dense weights, and the calls the int8 kernel does not take) merges its
 * waves' partial sums through LDS handshakes whose waits are bounded.  A wait that gives up
 * (which only a fault of the device could cause) is never silent: every give-up increments
 * a per-GPU device counter, and the outputs of a tile whose final wait gave up are stored
 * as NaN.
 *   qlin_merge_timeouts(reset): the current device's counter (call it after the launches
 *     have completed, e.g. once their stream is synchronized; it copies from the device);
 *     reset = 1 also clears it.  -1 on a HIP error or a reset other than 0 or 1.
 *   qlin_set_merge_spin_limit(limit): polls a wait makes before it gives up, for launches
 *     made after the call (default 4194304, each poll sleeping about 64 clocks); limit >= 0.
 *     A limit of 0 makes every wait give up at once, so that a test can see the report
 *     without any wait actually failing.  Returns the previous limit, or -1 (and changes
 *     nothing) for a negative limit.  Process-wide, not synchronized with other threads. */
int64_t qlin_merge_timeouts(int32_t reset);
int32_t qlin_set_merge_spin_limit(int32_t limit);

/* Static description of a status code. */
const char* qlin_status_string(qlin_status s);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
