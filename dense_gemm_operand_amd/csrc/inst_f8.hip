// Tiled-kernel instantiations for fp8 E4M3 operands (every layout pair), 256x256 tiles of
// eight waves, K step 128.
#include "kernels.hpp"

namespace dg {

static const Variant kTable[] = {
    // Defaults first (the planner takes the first match): the ping-pong schedule, with
    // direct-to-LDS loads for the K-contiguous operands (NN, TN, TT); NT has both operands
    // transposed in registers.
    TILE_LAYOUTS_PPDTL(F8T, 256, 256, 2, 4),
    TILE_PP(F8T, false, false, false, 256, 256, 2, 4, true, true),
    // the software-pipeline kernels (DGEMM_FORCE_SCHED=0)
    TILE_LAYOUTS_DTL(F8T, 256, 256, 2, 4),
    TILE(F8T, false, false, false, 256, 256, 2, 4, true),
};

int variants_f8(const Variant** out) {
  *out = kTable;
  return (int)(sizeof(kTable) / sizeof(kTable[0]));
}

}  // namespace dg
