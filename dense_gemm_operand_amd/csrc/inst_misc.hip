// Skinny split-K kernels, int4-B tiled kernels, identity-row-order comparison variants,
// and the dispatch over all instantiation tables.
#include <vector>

#include "kernels.hpp"

namespace dg {

static const Variant kTable[] = {
    // Skinny split-K kernels (M <= 16): (n-blocks of 16, waves, K iterations per register
    // set (two sets, so twice as many in flight), resident workgroups per CU assumed by the
    // split-K search). The first entry of a dtype is its default; the others are for tuning
    // (DGEMM_FORCE_SKINNY).
    SKINNY(F16T, false, 4, 4, 2, 2),
    SKINNY(BF16T, false, 4, 4, 2, 2),
    SKINNY(F16T, true, 2, 8, 2, 1),
    SKINNY(F16T, true, 4, 4, 2, 1),
    SKINNY(F16T, true, 2, 8, 4, 1),
    SKINNY(F16T, false, 4, 4, 1, 2),
    SKINNY(F16T, false, 4, 8, 2, 1),
    SKINNY(F16T, false, 2, 8, 2, 1),
    SKINNY(F16T, true, 4, 8, 2, 1),
    // int4 B (column-major codes), A either layout; row-major A: the ping-pong schedule with
    // A loaded straight into LDS (column-major A: the pipeline, which measured faster). The
    // 16x16x32 blocks keep their accumulators in VGPRs, which with the register-staged codes
    // and scales spilled and ran 2.1x slower; int4 B stays on 32x32x16 blocks.
    TILE_X(F16T, true, true, true, 256, 256, 2, 4, true, true, 1),
    TILE(F16T, true, true, true, 256, 256, 2, 4, true),
    TILE(F16T, false, true, true, 256, 256, 2, 4, true),
    TILE(F16T, true, true, true, 256, 256, 2, 2, true),
    TILE(F16T, false, true, true, 256, 256, 2, 2, true),
    TILE(F16T, true, true, true, 128, 128, 2, 2, true),
    TILE(F16T, false, true, true, 128, 128, 2, 2, true),
    // identity LDS row order (for comparisons of bank conflicts): padded rows, then
    // unpadded 128-byte rows
    TILE(F16T, false, true, false, 256, 256, 2, 4, 0),
    TILE(F16T, true, false, false, 256, 256, 2, 4, 0),
    TILE(F16T, false, true, false, 256, 256, 2, 2, 0),
    TILE(F16T, true, false, false, 256, 256, 2, 2, 0),
    TILE(BF16T, false, false, false, 256, 256, 2, 4, 0),
    TILE(F16T, false, true, false, 256, 256, 2, 4, 2),
    TILE(BF16T, false, false, false, 256, 256, 2, 4, 2),
};

int variants_misc(const Variant** out) {
  *out = kTable;
  return (int)(sizeof(kTable) / sizeof(kTable[0]));
}

namespace {
const std::vector<const Variant*>& all_variants() {
  static const std::vector<const Variant*> v = [] {
    std::vector<const Variant*> r;
    for (auto f : {variants_misc, variants_f16, variants_bf16, variants_f8}) {
      const Variant* t = nullptr;
      const int n = f(&t);
      for (int i = 0; i < n; ++i) r.push_back(t + i);
    }
    return r;
  }();
  return v;
}
}  // namespace

int variant_count() { return (int)all_variants().size(); }
const VariantInfo& variant_info(int i) { return all_variants()[i]->info; }

int launch(const Plan& p, const RunArgs& r, void* stream) {
  KArgs a;
  a.A = r.A;
  a.B = r.B;
  a.S = r.scales;
  a.C = r.C;
  a.counters = reinterpret_cast<int*>(r.ws);
  a.part = r.ws ? reinterpret_cast<float*>(reinterpret_cast<char*>(r.ws) + kCounterBytes) : nullptr;
  a.M = (int)p.M;
  a.N = (int)p.N;
  a.K = (int)p.K;
  a.ldA = (int)(p.layout_a == 0 ? p.K : p.M);
  a.ldB = (int)(p.layout_b == 0 ? p.N : p.K);
  const int64_t eb = p.dtype_a == DT_F8 ? 1 : 2;   // operand element bytes
  a.bytesA = (uint32_t)(p.M * p.K * eb);
  a.bytesB = (uint32_t)(p.dtype_b == DT_U4 ? p.N * p.K / 2 : p.N * p.K * eb);
  a.bytesS = (uint32_t)(p.dtype_b == DT_U4 ? (p.K >> p.group_log2) * p.N * 2 : 0);
  a.k_chunk = (int)p.k_chunk;
  a.tiles_m = (int)((p.M + p.tile_m - 1) / p.tile_m);
  a.tiles_n = (int)((p.N + p.tile_n - 1) / p.tile_n);
  a.dtype_c = p.dtype_c;
  const int ob = p.dtype_c == DT_F32 ? 4 : 2;
  a.c_vec = ((p.N * ob) % 16 == 0) ? 1 : 0;
  a.b_tiled = p.b_tiled;
  a.group_log2 = p.group_log2;
  a.zero = p.zero;
  if (p.kernel == KERNEL_SKINNY) a.c_vec = (p.N % 4 == 0) ? 1 : 0;  // 4-element stores
  return (int)all_variants()[p.variant]->fn(p, a, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace dg
