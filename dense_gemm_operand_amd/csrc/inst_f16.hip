// Tiled-kernel instantiations for fp16 operands (every layout pair).
#include "kernels.hpp"

namespace dg {

static const Variant kTable[] = {
    TILE_LAYOUTS(F16T, 256, 256, 2, 4),
    TILE_LAYOUTS(F16T, 256, 256, 2, 2),
    TILE_LAYOUTS(F16T, 192, 320, 2, 2),
    TILE_LAYOUTS(F16T, 128, 128, 2, 2),
};

int variants_f16(const Variant** out) {
  *out = kTable;
  return (int)(sizeof(kTable) / sizeof(kTable[0]));
}

}  // namespace dg
