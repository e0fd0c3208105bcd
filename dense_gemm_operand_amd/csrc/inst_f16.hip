// Tiled-kernel instantiations for fp16 operands (every layout pair).
#include "kernels.hpp"

namespace dg {

static const Variant kTable[] = {
    // Defaults first (the planner takes the first match): the 8-wave ping-pong schedule
    // with 16x16x32 blocks, K-contiguous operands straight into LDS; for NN the transposed
    // A through the in-register transpose; for TT and NT the transposed operands straight
    // into LDS in 64-wide K-row segments and transposed by the LDS reads (measured 2-3%
    // faster than the in-register transpose of TT's B, 11-18% faster than that of both of
    // NT's operands, DGEMM_FORCE_DTL=0). Then the alternatives: 32x32x16 blocks on the same
    // schedule (DGEMM_FORCE_MFMA=32), the single-schedule pipeline kernels
    // (DGEMM_FORCE_SCHED=0), NN with transposing reads (DGEMM_FORCE_DTL=2) and TT with the
    // in-register transpose (DGEMM_FORCE_DTL=1).
    TILE_XM(F16T, true, true, false, 256, 256, 2, 4, true, 1, 1, 16),
    TILE_XM(F16T, false, false, false, 256, 256, 2, 4, true, 1, 2, 16),
    TILE_XM(F16T, false, true, false, 256, 256, 2, 4, true, 1, 1, 16),
    TILE_XM(F16T, true, false, false, 256, 256, 2, 4, true, 1, 2, 16),
    TILE_LAYOUTS_PPDTL(F16T, 256, 256, 2, 4),
    TILE_LAYOUTS_PPTR(F16T, 256, 256, 2, 4),
    TILE_LAYOUTS_PP(F16T, 256, 256, 2, 4),
    TILE_LAYOUTS_DTL(F16T, 256, 256, 2, 4),
    TILE_LAYOUTS(F16T, 256, 256, 2, 4),
    TILE_LAYOUTS(F16T, 256, 256, 2, 2),
    // the non-power-of-2 192x320 tile (16 x 16 tiles for a 3072 x 5120 C on 256 CUs): first
    // the 8-wave ping-pong with 16x16x32 blocks (96x80 per wave) and every operand straight
    // into LDS (transposed ones in 64-wide K-row segments), then schedule 2 (4 waves), the
    // register-staged pipeline and the pipeline with direct loads
    TILE_LAYOUTS_PP16(F16T, 192, 320),
    TILE_LAYOUTS_W4(F16T, 192, 320),
    TILE_LAYOUTS(F16T, 192, 320, 2, 2),
    TILE_LAYOUTS_DTL(F16T, 192, 320, 2, 2),
    TILE_LAYOUTS_DTLTR(F16T, 192, 320, 2, 2),
    TILE_LAYOUTS(F16T, 128, 128, 2, 2),
    TILE_LAYOUTS(F16T, 64, 64, 2, 2),
    TILE_LAYOUTS_DTL(F16T, 256, 256, 2, 2),
    TILE_LAYOUTS_DTLTR(F16T, 256, 256, 2, 4),
    TILE_LAYOUTS_W4(F16T, 256, 256),
    TILE_XM(F16T, false, true, false, 256, 256, 2, 4, true, 1, 2, 16),
    TILE_XM(F16T, true, false, false, 256, 256, 2, 4, true, 1, 1, 16),
};

int variants_f16(const Variant** out) {
  *out = kTable;
  return (int)(sizeof(kTable) / sizeof(kTable[0]));
}

}  // namespace dg
