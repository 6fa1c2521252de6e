// Instantiations of the fused kernel for bf16 weights (one per activation-tile count).
#include "qlin_fused.h"

namespace qlin {

hipError_t launch_fused_bf16(const LinParams& p, int mt, int grid, size_t lds, hipStream_t s) {
  switch (mt) {
    case 1: return launch_one<16, true, 1>(p, grid, lds, s);
    case 2: return launch_one<16, true, 2>(p, grid, lds, s);
    case 3: return launch_one<16, true, 3>(p, grid, lds, s);
    case 4: return launch_one<16, true, 4>(p, grid, lds, s);
    case 5: return launch_one<16, true, 5>(p, grid, lds, s);
    case 6: return launch_one<16, true, 6>(p, grid, lds, s);
    case 7: return launch_one<16, true, 7>(p, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlin
