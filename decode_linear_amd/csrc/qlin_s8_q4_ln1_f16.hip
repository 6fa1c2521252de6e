// Instantiations of the int8 streaming kernel for 4-bit codes, LayerNorm on, f16
// activations (one unit per format, prologue and activation dtype, so that they compile in
// parallel).
#include "qlin_s8.h"

namespace qlin {
hipError_t launch_s8_q4_ln1_f16(const S8Launch& a, hipStream_t s) { return s8::launch_bits_ln<4, true, false>(a, s); }
}  // namespace qlin
