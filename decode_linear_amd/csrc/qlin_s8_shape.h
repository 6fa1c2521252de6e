// Launch description and shape limits of the int8 streaming kernel (qlin_s8.h), shared by
// the host code that chooses a launch and the kernel that runs it.
#pragma once

namespace qlin {

// Arguments of one launch of the int8 streaming kernel (qlin_s8.h), chosen by the host.
struct S8Launch {
  const void* x;                            // (T, K), fp16 or bf16
  const void* w0; const void* s0; const void* b0;   // codes, scales, biases (gate for gate/up)
  const void* p1; const void* p2; const void* p3;   // gate/up: up's codes, scales, biases; LN: gamma, beta
  int K, T, N, x_bf16, gateup, ln, bits;
  void* y; const void* res; const void* add;
  float eps;
  int y_dtype, act;
  int MT, GWM, D, waves, grid;   // D: tiles of the fullest workgroup
};
namespace s8 {
// Device addresses fit in the low 48 bits; the kernel's shape words ride above them.
constexpr int kTagShift = 48;
// Largest tile count a workgroup of this shape takes (VGPRs for the loads of every tile in
// flight at once, and LDS for their partials); 0 when the shape is not instantiated.  The
// shapes left out, and the one-tile limit of 8-bit windows of 16 groups, are those whose
// registers would spill (the build records every kernel's register use; a test checks that
// no instantiated shape spills).
constexpr int max_tiles(int bits, bool ln, int mt, int gwm) {
  return mt == 1 ? (gwm <= 8 ? 8 : gwm == 16 ? (bits == 8 ? 1 : 8) : gwm == 32 ? (ln ? 0 : 1) : 0)
       : mt == 2 ? (gwm <= 4 ? 8 : (gwm == 8 ? 4 : 0))
       : mt == 3 ? (gwm <= 4 ? 4 : 0)
       : mt == 9 ? (gwm == 2 ? 1 : 0) : 0;
}
// Shapes with a one-tile, 16-wave instantiation (a long K over more waves).
constexpr bool wide_ok(int bits, bool ln, int mt, int gwm) {
  return mt == 1 ? (gwm == 4 || gwm == 8 || (gwm == 16 && bits == 4 && !ln)) : (mt == 2 && gwm == 4);
}
// Workgroups of more than one tile keep two ring slots (launch_d): the next tile's loads
// are in flight while the wave computes.  Deeper rings measured slower on the SwiGLU workload (3 and 4
// slots: 18.2 and 17.3 against 17.0 us): with more requests outstanding the weight
// stream's rate drops.
}  // namespace s8
}  // namespace qlin
