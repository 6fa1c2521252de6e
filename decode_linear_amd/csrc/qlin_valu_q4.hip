// Instantiations of the vector-ALU streaming kernel (qlin_valu.h) for 4-bit codes.
#include "qlin_valu.h"

namespace qlin {
hipError_t launch_valu_q4(const S8Launch& a, hipStream_t s) {
  return a.ln ? va::launch_bits_ln<4, true>(a, s) : va::launch_bits_ln<4, false>(a, s);
}
}  // namespace qlin
