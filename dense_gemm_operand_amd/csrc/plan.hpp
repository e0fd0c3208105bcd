// Internal plan record shared by the planner, the ABI layer and the kernel launchers.
#pragma once
#include <cstdint>

namespace dg {

enum Kernel : int32_t { KERNEL_TILE = 0, KERNEL_SKINNY = 1 };

// Element-type codes (same numbering as the public header).
enum Dtype : int32_t { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_U4 = 3, DT_F8 = 4 };

struct Plan {
  int64_t M = 0, N = 0, K = 0;
  int32_t layout_a = 0, layout_b = 0;  // 0 row-major, 1 column-major
  int32_t dtype_a = 0, dtype_b = 0, dtype_c = 0;
  int32_t kernel = KERNEL_TILE;
  int32_t variant = -1;                // index into the launcher's instantiation table
  int32_t tile_m = 0, tile_n = 0, tile_k = 0;
  int32_t waves = 0;
  int32_t lds_pad = 0, perm_block = 1, perm_stride = 1;
  int32_t split_k = 1;                 // across workgroups
  int32_t wave_split_k = 1;            // across waves of a workgroup
  int64_t k_chunk = 0;                 // K elements per split (multiple of the step)
  int64_t grid_x = 0, grid_y = 0, grid_z = 0;
  int64_t tiles = 0;                   // output tiles (= counters used when split_k > 1)
  int64_t partial_bytes_per_split = 0; // fp32 partial bytes of one split
  int64_t workspace_bytes = 0;
  int32_t lds_bytes = 0;
  int32_t cu_count = 0;
  int32_t slots_per_cu = 1;
  int32_t direct_lds = 0;              // bit 0: A, bit 1: B loaded straight into LDS
  int32_t b_tiled = 0;                 // int4 codes in the pre-tiled layout (layout_b 2)
  int32_t group_log2 = 7;              // int4: log2 of the scale group size
  int32_t zero = 8;                    // int4: zero point
  int32_t device = -1;
};

// Arrival counters occupy the first kCounterBytes of every workspace.
constexpr int64_t kCounterBytes = 64 * 1024;
constexpr int64_t kMaxCounters = kCounterBytes / 4;

// Device pointers and sizes for one run.
struct RunArgs {
  const void* A;
  const void* B;
  const void* scales;
  void* C;
  void* ws;
};

// Instantiation table of the launcher (kernels.hip).
struct VariantInfo {
  int32_t kernel;
  int32_t dtype_a, dtype_b;       // DT_F16/DT_BF16/DT_F8; dtype_b DT_U4 for int4
  int32_t layout_a, layout_b;     // required layouts
  int32_t tile_m, tile_n, tile_k;
  int32_t waves;
  int32_t wave_split_k;
  int32_t perm;                   // LDS rows of thread-stored operands: 1 = permuted (transposed
                                  // operands) and padded, 0 = identity order, padded, 2 = identity
                                  // order, unpadded
  int32_t lds_bytes;
  int32_t depth;                  // skinny: K iterations in flight per wave
  int32_t slots_per_cu;           // workgroups assumed resident per CU by the split-K search
  int32_t sched;                  // tiled: 0 = software pipeline, 1 = ping-pong wave groups
  int32_t dtl;                    // tiled: bit 0 A, bit 1 B loaded straight into LDS;
                                  // bit 2 A, bit 3 B transposed by the LDS reads
  int32_t mfma;                   // matrix-core block: 32 (32x32x16 / 32x32x64) or 16 (16x16x32)
};

// One attention forward call (validated by the ABI layer).
struct AttnLaunch {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int64_t BH, Sq, Sk, D;
  int32_t dtype;
  float scale;
};
// Returns 0 or a hipError_t value.
int launch_attn(const AttnLaunch& l, void* stream);

int variant_count();
const VariantInfo& variant_info(int i);
// Returns 0 or a hipError_t value.
int launch(const Plan& p, const RunArgs& a, void* stream);

}  // namespace dg
