// Instantiations of the int8 streaming kernel for 8-bit codes, LayerNorm off, f16
// activations (one unit per format, prologue and activation dtype, so that they compile in
// parallel).
#include "qlin_s8.h"

namespace qlin {
hipError_t launch_s8_q8_ln0_f16(const S8Launch& a, hipStream_t s) { return s8::launch_bits_ln<8, false, false>(a, s); }
}  // namespace qlin
