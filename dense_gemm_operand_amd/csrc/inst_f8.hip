// Tiled-kernel instantiations for fp8 E4M3 operands (every layout pair), 256x256 tiles of
// eight waves, K step 128.
#include "kernels.hpp"

namespace dg {

static const Variant kTable[] = {
    // direct-to-LDS loads for the K-contiguous operands (NN, TN, TT)
    TILE_LAYOUTS_DTL(F8T, 256, 256, 2, 4),
    // both operands transposed in registers (NT)
    TILE(F8T, false, false, false, 256, 256, 2, 4, true),
};

int variants_f8(const Variant** out) {
  *out = kTable;
  return (int)(sizeof(kTable) / sizeof(kTable[0]));
}

}  // namespace dg
