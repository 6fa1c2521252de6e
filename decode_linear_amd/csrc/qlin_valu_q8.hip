// Instantiations of the vector-ALU streaming kernel (qlin_valu.h) for 8-bit codes.
#include "qlin_valu.h"

namespace qlin {
hipError_t launch_valu_q8(const S8Launch& a, hipStream_t s) {
  return a.ln ? va::launch_bits_ln<8, true>(a, s) : va::launch_bits_ln<8, false>(a, s);
}
}  // namespace qlin
