// Instantiations of the fused kernel for q4 weights (one per activation-tile count).
#include "qlin_fused.h"

namespace qlin {

hipError_t launch_fused_q4(const LinParams& p, int mt, int grid, size_t lds, hipStream_t s) {
  switch (mt) {
    case 1: return launch_one<4, false, 1>(p, grid, lds, s);
    case 2: return launch_one<4, false, 2>(p, grid, lds, s);
    case 3: return launch_one<4, false, 3>(p, grid, lds, s);
    case 4: return launch_one<4, false, 4>(p, grid, lds, s);
    case 5: return launch_one<4, false, 5>(p, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlin
