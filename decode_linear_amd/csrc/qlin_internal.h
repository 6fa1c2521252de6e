// Internal interface between libqlin's host code (qlin_host.cpp) and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_s8_shape.h"

namespace qlin {

// Waves per workgroup of the fused kernel.  Each wave owns a fixed slice of K and keeps
// its activation fragments in registers; the workgroup merges the slices in LDS.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

// Arguments of one fused-linear launch (plain linear or gate/up).
struct LinParams {
  const void* x;          // (T, K) activations, x_dtype
  int x_dtype;            // 1 fp16, 2 bf16
  int T, K, N;
  const void* w[2];       // weight rows (gate in w[0], up in w[1] for gate/up)
  const uint16_t* sc[2];  // fp16 scales (N, K/64), quantized only
  const uint16_t* bi[2];  // fp16 biases
  int gateup;             // 0: y = epi(z); 1: y = silu(z_gate) * z_up
  int ln;                 // LayerNorm prologue on/off
  const void* gamma;
  const void* beta;
  float eps;
  int terms;              // 16-bit operand terms per activation row (1, 2 or 3)
  int scale_act;          // 1: scale activation rows into the binary16 range per wave
  int scale_gb;           // 1: same for the gamma / beta rows
  int act;                // 0 none, 1 GELU
  const void* res;        // (T, N) or null
  const void* add;        // (N,) or null
  void* y;                // (T, N)
  int y_dtype;            // 0 fp32, 1 fp16, 2 bf16
  int rows;               // operand rows: terms*T (+ gamma, beta with LN)
  int ntiles;             // 16-column output tiles (linear) or 8-column tiles (gate/up)
  int steps;              // 64-byte steps per weight row
  int chunk_steps;        // steps staged at once (all of them unless K is long)
  int spin;               // polls a merge wait makes before it gives up
  unsigned int* timeouts; // device counter of merge waits that gave up
};

// Rows of the activation operand: terms*T activation terms, then gamma and beta (LN).
inline int act_rows(int T, int terms, int ln) { return terms * T + (ln ? 2 : 0); }

// Launchers (one per weight format / operand type), defined in the kernel sources.
// mt = number of 16-row activation tiles (1..7).  Return the launch error.
hipError_t launch_fused_q4(const LinParams& p, int mt, int grid, size_t lds, hipStream_t s);
hipError_t launch_fused_q8(const LinParams& p, int mt, int grid, size_t lds, hipStream_t s);
hipError_t launch_fused_f16(const LinParams& p, int mt, int grid, size_t lds, hipStream_t s);
hipError_t launch_fused_bf16(const LinParams& p, int mt, int grid, size_t lds, hipStream_t s);
// Steps staged per chunk for this shape (all steps when the operand fits in registers and
// LDS) and the dynamic LDS bytes the launch needs.
int fused_chunk_steps(int bits, int mt, int T, int ln, int rows, long K);
size_t fused_lds_bytes(int bits, int rows, int chunk_steps, long K, int mt);

// One launcher per code width and prologue (qlin_s8_q{4,8}_ln{0,1}.hip).
hipError_t launch_s8_q4_ln0_bf16(const S8Launch& a, hipStream_t s);
hipError_t launch_s8_q4_ln0_f16(const S8Launch& a, hipStream_t s);
hipError_t launch_s8_q4_ln1_bf16(const S8Launch& a, hipStream_t s);
hipError_t launch_s8_q4_ln1_f16(const S8Launch& a, hipStream_t s);
hipError_t launch_s8_q8_ln0_bf16(const S8Launch& a, hipStream_t s);
hipError_t launch_s8_q8_ln0_f16(const S8Launch& a, hipStream_t s);
hipError_t launch_s8_q8_ln1_bf16(const S8Launch& a, hipStream_t s);
hipError_t launch_s8_q8_ln1_f16(const S8Launch& a, hipStream_t s);
// The vector-ALU streaming kernel for T <= 4 (qlin_valu.h): S8Launch with MT = activation
// rows held (1, 2 or 4) and GWM = lanes per weight row (16 or 32).
hipError_t launch_valu_q4(const S8Launch& a, hipStream_t s);
hipError_t launch_valu_q8(const S8Launch& a, hipStream_t s);
hipError_t launch_valu_f16(const S8Launch& a, hipStream_t s);   // dense fp16 weights and activations

// Arguments of one attend launch (cache append + causal attention, <= 32 positions).
struct AttendParams {
  const void* qkv;        // (T, 3 * H * HD), dtype
  const void* kv;         // (2, H, P, HD), dtype; null when P == 0
  void* out;              // (T, H * HD) or (1, H * HD) with last, out_dtype
  void* kv_out;           // (2, H, P + T, HD), dtype
  int dtype;              // 1 fp16, 2 bf16
  int out_dtype;          // 0 fp32, 1 fp16, 2 bf16
  int H, HD, P, T;
  int last;               // 1: only the last new position's output row
  float scale;            // 1 / sqrt(HD), rounded to fp32
};
hipError_t launch_attend(const AttendParams& a, hipStream_t s);

hipError_t launch_pack(const float* w, int64_t N, int64_t K, int bits, uint32_t* codes, uint16_t* scales,
                       uint16_t* biases, int32_t* flag, hipStream_t s);
hipError_t launch_unpack(const void* data, const uint16_t* scales, const uint16_t* biases, int bits,
                         int dtype, int64_t N, int64_t K, float* out, hipStream_t s);

// Arguments of one sample launch (exact top-k, Gumbel-max, embedding append).
constexpr int kSampleMaxCodes = 8192;
struct SampleParams {
  const void* logits;     // (n) of logit_dtype
  int logit_dtype;        // 0 fp32, 1 fp16, 2 bf16
  int n;                  // 1 .. kSampleMaxCodes
  const float* gumbel;    // (n) this level's noise
  float inv_temp;
  int top_k;              // 1 .. n
  const void* table;      // (n, D) this level's embeddings, or null
  const void* prefix;     // (n_prev, D), or null when n_prev == 0
  int n_prev, D, es;      // rows, row width, element bytes (D * es a multiple of 16)
  void* out;              // (n_prev + (table != null), D)
  int32_t* code;          // (1)
  int copy_prefix;        // 0: out is the prefix itself (append in place)
};
hipError_t launch_sample(const SampleParams& a, hipStream_t s);

// Arguments of one quantized-KV decode attention (block partials + merge).
struct KvqParams {
  const void* q;            // (H, D), q_dtype
  int q_dtype;              // 1 fp16, 2 bf16
  int q_vec;                // 1: q is 16-byte aligned (read with 16-byte loads)
  const uint32_t* kc;       // (KV, N, D * bits / 32)
  const void* ks;           // (KV, N, D / GS), sb_dtype
  const void* kb;
  const uint32_t* vc;
  const void* vs;
  const void* vb;
  int sb_dtype;             // 1 fp16, 2 bf16
  int H, KV, N, D, GS, bits;
  int block, G;             // rows per block, blocks
  float* opart;             // (H, G, D) workspace
  float* stats;             // (H, G, 2) workspace: block max, block sum
  void* out;                // (H, D), out_dtype
  int out_dtype;            // 0 fp32, 1 fp16, 2 bf16
};
hipError_t launch_kvq_decode(const KvqParams& a, hipStream_t s);
// Device address, on the current device, of the static scratch array behind
// qlin_kvq_decode_noalloc (QLIN_KVQ_SCRATCH_BYTES); looked up once per device.
hipError_t kvq_scratch(float** ptr);

// Plain 16-byte streaming read of `bytes` (a multiple of 16) at buf; block b writes the XOR
// fold of the words it read to partial[b] (grid blocks of 512 threads, `unroll` loads in
// flight per thread: 1, 2, 4, 8 or 16; non-temporal loads when nt).
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* partial, int grid, int unroll, bool nt,
                              hipStream_t s);

}  // namespace qlin
