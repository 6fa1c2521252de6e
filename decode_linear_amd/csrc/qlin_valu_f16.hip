// Instantiations of the vector-ALU streaming kernel (qlin_valu.h) for dense fp16 weights.
#include "qlin_valu.h"

namespace qlin {
hipError_t launch_valu_f16(const S8Launch& a, hipStream_t s) {
  return a.ln ? va::launch_bits_ln<16, true>(a, s) : va::launch_bits_ln<16, false>(a, s);
}
}  // namespace qlin
