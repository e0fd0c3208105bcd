// Host side of libdgemm: argument validation, the planner and the extern "C" entry points
// declared in include/dgemm.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <new>

#include "../../include/dattn.h"
#include "../../include/dgemm.h"
#include "lds_layout.hpp"
#include "plan.hpp"

struct gemm_plan_s {
  dg::Plan p;
};

namespace dg {
namespace {

bool debug_on() { return std::getenv("DGEMM_DEBUG") != nullptr; }

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split-K factor: BitBLAS PR 268, "SplitK Infer". Start at 1; with grid = tiles * factor,
// the waste is grid mod num_cus and the ratio waste / grid; stop once the ratio is at most
// 5%, else double the factor unless the doubled factor times the K step reaches K. Tile
// counts use ceiling division (a floor would leave an empty grid when a tile is taller
// than M); the factor is capped at 16.
int splitk_search(int64_t tiles, int64_t K, int64_t k_step, int num_cus) {
  int f = 1;
  for (;;) {
    const int64_t grid = tiles * f;
    const int64_t waste = grid - (grid / num_cus) * num_cus;
    if ((double)waste / (double)grid <= 5e-2) break;
    const int nxt = f * 2;
    if ((int64_t)nxt * k_step >= K || nxt > 16) break;
    f = nxt;
  }
  return f;
}

int cu_count_for(int* device, int* status) {
  *status = GEMM_OK;
  const int fake = env_int("DGEMM_FAKE_CU_COUNT", 0);
  if (fake > 0) {
    *device = -1;
    return fake;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *status = GEMM_ERR_NO_DEVICE;
    return 0;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    *status = GEMM_ERR_NO_DEVICE;
    return 0;
  }
  *device = dev;
  return prop.multiProcessorCount;
}

// Candidate matching the request, or -1.
int find_variant(int kernel, const Plan& p, int tm, int tn, int perm) {
  // DGEMM_FORCE_WAVES=<n> restricts tiled variants to n waves per workgroup (tuning).
  const int waves = env_int("DGEMM_FORCE_WAVES", 0);
  for (int i = 0; i < variant_count(); ++i) {
    const VariantInfo& v = variant_info(i);
    if (kernel == KERNEL_TILE && waves > 0 && v.waves != waves) continue;
    // DGEMM_FORCE_SCHED=<0|1|2> restricts tiled variants to one main-loop schedule: 0 software
    // pipeline, 1 two-group ping-pong, 2 four waves with every operand loaded straight into
    // LDS (tuning, tests).
    const int sched = env_int("DGEMM_FORCE_SCHED", -1);
    if (kernel == KERNEL_TILE && sched >= 0 && v.sched != sched) continue;
    // DGEMM_FORCE_DTL=<0|1|2> restricts tiled variants to ones without direct-to-LDS loads,
    // with them for K-contiguous operands only, or with them for transposed operands too
    // (transposed by the LDS reads) (tuning, tests).
    const int dtl = env_int("DGEMM_FORCE_DTL", -1);
    // DGEMM_FORCE_MFMA=<32|16> restricts tiled variants to one matrix-core block (tests).
    const int mfma = env_int("DGEMM_FORCE_MFMA", 0);
    if (kernel == KERNEL_TILE && mfma > 0 && v.mfma != mfma) continue;
    const int have = (v.dtl & 12) ? 2 : (v.dtl ? 1 : 0);
    if (kernel == KERNEL_TILE && dtl >= 0 && have != dtl) continue;
    if (v.kernel != kernel || v.dtype_a != p.dtype_a || v.dtype_b != p.dtype_b) continue;
    if (kernel == KERNEL_TILE) {
      if (v.layout_a != p.layout_a || v.layout_b != p.layout_b) continue;
      if (v.tile_m != tm || v.tile_n != tn || v.perm != perm) continue;
    } else {
      if (v.layout_a != p.layout_a || v.layout_b != p.layout_b) continue;
      // DGEMM_FORCE_SKINNY=<n-blocks>x<waves>x<depth> picks one skinny variant (tuning).
      int nb = 0, w = 0, d = 0;
      if (const char* fs = std::getenv("DGEMM_FORCE_SKINNY")) {
        std::sscanf(fs, "%dx%dx%d", &nb, &w, &d);
        if (v.tile_n != 16 * nb || v.waves != w || v.depth != d) continue;
      }
    }
    return i;
  }
  return -1;
}

int make_plan(Plan& p, int split_k_req) {
  int status = GEMM_OK;
  p.cu_count = cu_count_for(&p.device, &status);
  if (status != GEMM_OK) return status;

  const int forced = env_int("DGEMM_FORCE_VARIANT", -1);
  // DGEMM_NO_PERM=1 takes the variant with identity LDS row order, =2 the one with identity
  // order and unpadded 128-byte rows (comparison variants for bank-conflict measurements).
  const int no_perm = env_int("DGEMM_NO_PERM", 0);
  const int lrows = no_perm == 2 ? 2 : (no_perm ? 0 : 1);
  int vi = -1;
  if (forced >= 0) {
    if (forced >= variant_count()) return GEMM_ERR_INVALID_ARG;
    const VariantInfo& v = variant_info(forced);
    if (v.dtype_a != p.dtype_a || v.dtype_b != p.dtype_b || v.layout_a != p.layout_a ||
        v.layout_b != p.layout_b || (v.kernel == KERNEL_SKINNY && p.M > 16))
      return GEMM_ERR_UNSUPPORTED;
    vi = forced;
  } else {
    // Skinny kernel: at most 16 rows, K-contiguous operands (TN) or int4 B.
    if (p.M <= 16 && !std::getenv("DGEMM_FORCE_TILE")) vi = find_variant(KERNEL_SKINNY, p, 0, 0, 0);
    if (vi < 0) {
      // Tiled kernel: among the instantiated tiles, the one with the least work per CU,
      // i.e. ceil(tiles / CUs) * tile area (larger tiles first on ties). A 4-wave tile is
      // charged 5/4 of its area: measured per tile area it runs about that much slower than
      // the 8-wave 256x256 kernels (one wave per SIMD hides less latency).
      static const int kTiles[][2] = {{256, 256}, {192, 320}, {128, 128}, {64, 64}};
      // DGEMM_FORCE_TILE=<m>x<n> restricts the choice to one tile (tests, tuning).
      int force_m = 0, force_n = 0;
      if (const char* ft = std::getenv("DGEMM_FORCE_TILE")) std::sscanf(ft, "%dx%d", &force_m, &force_n);
      int64_t best = -1;
      for (const auto& t : kTiles) {
        if (force_m > 0 && (t[0] != force_m || t[1] != force_n)) continue;
        const int v = find_variant(KERNEL_TILE, p, t[0], t[1], lrows);
        if (v < 0) continue;
        const int64_t tiles = cdiv(p.M, t[0]) * cdiv(p.N, t[1]);
        const int64_t cost = cdiv(tiles, p.cu_count) * t[0] * t[1] * (variant_info(v).waves >= 8 ? 4 : 5);
        if (best < 0 || cost < best) {
          best = cost;
          vi = v;
        }
      }
    }
  }
  if (vi < 0) return GEMM_ERR_UNSUPPORTED;
  const VariantInfo& v = variant_info(vi);
  p.variant = vi;
  p.kernel = v.kernel;
  p.tile_m = v.tile_m;
  p.tile_n = v.tile_n;
  p.tile_k = v.tile_k;
  p.waves = v.waves;
  p.wave_split_k = v.wave_split_k;
  // padding after each row of an operand stored by the threads: 16 bytes, 32 for the 16x16x32
  // kernels (whose transposed rows also swap chunk c to c ^ ((r >> 2) & 1))
  p.lds_pad = (v.kernel == KERNEL_TILE && v.mfma == 16) ? 32 : 16;
  const bool transposed = (p.layout_a == 1) || (p.layout_b == 0 && p.dtype_b != DT_U4);
  // row permutation of operands transposed in registers: 64 rows, stride 8 (16-bit) or
  // 256 rows, stride 16 (fp8)
  const bool f8 = p.dtype_a == DT_F8;
  p.perm_block = (v.kernel == KERNEL_TILE && v.perm == 1 && transposed) ? (f8 ? 256 : 64) : 1;
  p.perm_stride = p.perm_block > 1 ? (f8 ? 16 : 8) : 1;
  p.lds_bytes = v.lds_bytes;
  p.slots_per_cu = v.slots_per_cu;
  p.direct_lds = v.kernel == KERNEL_TILE ? v.dtl : 0;
  if (p.direct_lds == 3) p.lds_pad = 0;  // neither operand is stored by the threads
  if (v.kernel == KERNEL_TILE && v.perm == 2) p.lds_pad = 0;  // unpadded comparison variant
  if (p.direct_lds & 12) {
    // transposed operands in global order: 64 bytes of padding per 1 KiB LDS block and the
    // K-row permutation B = 8, S = 4 (256-wide tiles, two K rows per block) or B = 64,
    // S = 8 (other widths, eight 64-wide K-row segments per block)
    const int tr_rows = (p.direct_lds & 4) ? p.tile_m : p.tile_n;
    const bool two_rows = tr_rows == 256 && v.mfma == 32;
    p.lds_pad = 64;
    p.perm_block = two_rows ? 8 : 64;
    p.perm_stride = two_rows ? 4 : 8;
  }
  if (v.kernel == KERNEL_SKINNY) {
    p.lds_pad = 0;
    p.lds_bytes = v.waves * (v.tile_n / 16) * 64 * 16;
  }

  const int64_t tiles = cdiv(p.M, p.tile_m) * cdiv(p.N, p.tile_n);
  p.tiles = tiles;
  // K granule of one split: the main-loop step (tiled) or one step per wave (skinny).
  const int64_t k_step = v.kernel == KERNEL_TILE ? v.tile_k : (int64_t)v.tile_k * v.waves;
  int sk = split_k_req;
  const int forced_sk = env_int("DGEMM_FORCE_SPLIT_K", 0);
  if (forced_sk > 0) sk = forced_sk;
  // The search counts workgroup slots: CUs times the workgroups the variant keeps
  // resident per CU (the skinny kernels are small enough for two).
  if (sk == 0) sk = splitk_search(tiles, p.K, k_step, p.cu_count * v.slots_per_cu);
  if (sk > 1 && tiles > kMaxCounters) sk = 1;
  // schedule 2 (4 waves of 128x128 accumulators) has no split-K fix-up
  if (v.kernel == KERNEL_TILE && v.sched == 2) sk = 1;
  p.split_k = sk;
  // chunk: ceil(K / sk) rounded up to the per-iteration granule of the kernel
  // int4 splits start on a multiple of 128 K (one skinny-kernel iteration, one block of the
  // pre-tiled code layout); scales are looked up by absolute K, so any group size works
  const int64_t gran = p.dtype_b == DT_U4 ? 128 : v.tile_k;
  p.k_chunk = cdiv(cdiv(p.K, sk), gran) * gran;
  if (v.kernel == KERNEL_TILE) {
    p.grid_x = tiles;
    p.grid_y = 1;
    p.grid_z = sk;
  } else {
    p.grid_x = tiles;
    p.grid_y = sk;
    p.grid_z = 1;
  }
  // fp32 partial tile as the kernels store it: the whole tile (the tiled kernel's
  // accumulators, the skinny kernel's reduced tile of 16 x tile_n fp32 values, which its
  // threads own in whole four-value positions)
  const int64_t per_tile = (int64_t)(v.kernel == KERNEL_SKINNY ? 16 : p.tile_m) * p.tile_n * 4;
  p.partial_bytes_per_split = tiles * per_tile;
  p.workspace_bytes = sk > 1 ? kCounterBytes + (int64_t)sk * p.partial_bytes_per_split : 0;
  if (debug_on())
    std::fprintf(stderr, "[dgemm] plan M=%lld N=%lld K=%lld variant=%d tile=%dx%d sk=%d\n",
                 (long long)p.M, (long long)p.N, (long long)p.K, vi, p.tile_m, p.tile_n, sk);
  return GEMM_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace
}  // namespace dg

extern "C" {

int gemm_plan(gemm_plan_t* out, int64_t M, int64_t N, int64_t K, int layout_a, int layout_b,
              int dtype_a, int dtype_b, int dtype_c, int split_k, const gemm_quant_t* quant) {
  using namespace dg;
  if (!out) return GEMM_ERR_INVALID_ARG;
  *out = nullptr;
  if (M <= 0 || N <= 0 || K <= 0) return GEMM_ERR_INVALID_ARG;
  if ((layout_a != 0 && layout_a != 1) || (layout_b < 0 || layout_b > 2))
    return GEMM_ERR_INVALID_ARG;
  const bool b_tiled = layout_b == 2;
  if (b_tiled && (dtype_b != DT_U4 || N % 64 != 0)) return GEMM_ERR_UNSUPPORTED;
  if (dtype_a < 0 || dtype_a > 4 || dtype_b < 0 || dtype_b > 4 || dtype_c < 0 || dtype_c > 4)
    return GEMM_ERR_INVALID_ARG;
  if (split_k < 0) return GEMM_ERR_INVALID_ARG;
  if (split_k != 0 && split_k != 1 && split_k != 2 && split_k != 4 && split_k != 8 &&
      split_k != 16)
    return GEMM_ERR_UNSUPPORTED;
  if (dtype_a != DT_F16 && dtype_a != DT_BF16 && dtype_a != DT_F8) return GEMM_ERR_UNSUPPORTED;
  if (dtype_c == DT_U4 || dtype_c == DT_F8) return GEMM_ERR_UNSUPPORTED;
  if (dtype_b == DT_U4) {
    if (dtype_a != DT_F16 || layout_b == 0 || !quant) return GEMM_ERR_UNSUPPORTED;
    // group: a power of two from 32 to K dividing K; zero point 0..15
    const int64_t g = quant->group_size;
    if (g < 32 || (g & (g - 1)) != 0 || g > K || K % g != 0 || quant->zero_point < 0 ||
        quant->zero_point > 15 || quant->scale_dtype != DT_F16 || quant->scale_layout != 0)
      return GEMM_ERR_UNSUPPORTED;
    if (K % 128 != 0) return GEMM_ERR_UNSUPPORTED;
  } else if (dtype_b != dtype_a) {
    return GEMM_ERR_UNSUPPORTED;
  }
  // 32-bit buffer offsets: every operand below 2 GiB, every size within int range. Each
  // extent is bounded first, so that no product below can overflow; the byte limits are
  // then compared as element counts (lim - 16 and lim divide by eb and ob).
  const int64_t lim = (int64_t)1 << 31;
  const int64_t eb = dtype_a == DT_F8 ? 1 : 2;
  const int64_t ob = dtype_c == DT_F32 ? 4 : 2;
  if (M >= lim || N >= lim || K >= lim) return GEMM_ERR_UNSUPPORTED;
  // contiguous extents: multiples of 16 bytes (8 16-bit or 16 fp8 elements)
  const int64_t ca = layout_a == 0 ? K : M;
  const int64_t cb = dtype_b == DT_U4 ? K : (layout_b == 0 ? N : K);
  if ((ca * eb) % 16 != 0 || (cb * eb) % 16 != 0) return GEMM_ERR_UNSUPPORTED;
  if (M * K >= (lim - 16) / eb || N * K >= (lim - 16) / eb || M * N >= lim / ob)
    return GEMM_ERR_UNSUPPORTED;

  gemm_plan_s* h = new (std::nothrow) gemm_plan_s;
  if (!h) return GEMM_ERR_INVALID_ARG;
  Plan& p = h->p;
  p.M = M;
  p.N = N;
  p.K = K;
  p.layout_a = layout_a;
  p.layout_b = b_tiled ? 1 : layout_b;   // the tiled codes are K-packed like column-major
  p.b_tiled = b_tiled ? 1 : 0;
  p.dtype_a = dtype_a;
  p.dtype_b = dtype_b;
  p.dtype_c = dtype_c;
  if (dtype_b == DT_U4) {
    int lg = 0;
    while ((int64_t)1 << lg < quant->group_size) ++lg;
    p.group_log2 = lg;
    p.zero = quant->zero_point;
  }
  const int st = make_plan(p, split_k);
  if (st != GEMM_OK) {
    delete h;
    return st;
  }
  *out = h;
  return GEMM_OK;
}

int gemm_pack_u4_tiled(const void* codes, void* tiled, int64_t N, int64_t K) {
  if (!codes || !tiled || N <= 0 || K <= 0) return GEMM_ERR_INVALID_ARG;
  if (N % 64 != 0 || K % 128 != 0) return GEMM_ERR_UNSUPPORTED;
  const uint8_t* src = static_cast<const uint8_t*>(codes);
  uint8_t* dst = static_cast<uint8_t*>(tiled);
  const int64_t groups = K / 128;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < groups; ++g)
      std::memcpy(dst + ((n / 64) * groups + g) * 4096 + (n % 64) * 64, src + n * (K / 2) + g * 64, 64);
  return GEMM_OK;
}

int gemm_workspace_size(gemm_plan_t plan, size_t* bytes) {
  if (!plan || !bytes) return GEMM_ERR_INVALID_ARG;
  *bytes = (size_t)plan->p.workspace_bytes;
  return GEMM_OK;
}

int gemm_run(gemm_plan_t plan, const void* A, const void* B, const void* scales, void* C,
             void* workspace, size_t ws_bytes, void* stream) {
  using namespace dg;
  if (!plan || !A || !B || !C) return GEMM_ERR_INVALID_ARG;
  const Plan& p = plan->p;
  if (p.dtype_b == DT_U4 && !scales) return GEMM_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (scales && !aligned16(scales)))
    return GEMM_ERR_MISALIGNED;
  if (p.workspace_bytes > 0) {
    if (!workspace) return GEMM_ERR_INVALID_ARG;
    if (!aligned16(workspace)) return GEMM_ERR_MISALIGNED;
    if (ws_bytes < (size_t)p.workspace_bytes) return GEMM_ERR_WORKSPACE_TOO_SMALL;
  }
  if (p.device < 0) return GEMM_ERR_NO_DEVICE;  // planned without a device
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != p.device) return GEMM_ERR_NO_DEVICE;
  RunArgs r{A, B, scales, C, p.workspace_bytes > 0 ? workspace : nullptr};
  const int e = launch(p, r, stream);
  if (e != 0) {
    if (debug_on()) std::fprintf(stderr, "[dgemm] launch failed: %s\n", hipGetErrorString((hipError_t)e));
    return GEMM_ERR_HIP;
  }
  return GEMM_OK;
}

int gemm_plan_query(gemm_plan_t plan, gemm_plan_info_t* info) {
  if (!plan || !info) return GEMM_ERR_INVALID_ARG;
  const dg::Plan& p = plan->p;
  std::memset(info, 0, sizeof(*info));
  info->M = p.M;
  info->N = p.N;
  info->K = p.K;
  info->layout_a = p.layout_a;
  info->layout_b = p.b_tiled ? 2 : p.layout_b;
  info->dtype_a = p.dtype_a;
  info->dtype_b = p.dtype_b;
  info->dtype_c = p.dtype_c;
  info->kernel = p.kernel;
  info->tile_m = p.tile_m;
  info->tile_n = p.tile_n;
  info->tile_k = p.tile_k;
  info->waves = p.waves;
  info->lds_pad_bytes = p.lds_pad;
  info->perm_block = p.perm_block;
  info->perm_stride = p.perm_stride;
  info->split_k = p.split_k;
  info->wave_split_k = p.wave_split_k;
  info->grid_x = p.grid_x;
  info->grid_y = p.grid_y;
  info->grid_z = p.grid_z;
  info->workspace_bytes = p.workspace_bytes;
  info->lds_bytes = p.lds_bytes;
  info->cu_count = p.cu_count;
  info->slots_per_cu = p.slots_per_cu;
  info->direct_lds = p.direct_lds;
  info->schedule = p.kernel == dg::KERNEL_TILE ? dg::variant_info(p.variant).sched : 0;
  info->mfma_m = dg::variant_info(p.variant).mfma;
  return GEMM_OK;
}

void gemm_plan_destroy(gemm_plan_t plan) { delete plan; }

const char* gemm_status_string(int status) {
  switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_ERR_UNSUPPORTED: return "unsupported request";
    case GEMM_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case GEMM_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GEMM_ERR_NO_DEVICE: return "no usable HIP device";
    case GEMM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int attn_fwd(const void* Q, const void* K, const void* V, void* O, int64_t BH, int64_t Sq,
             int64_t Sk, int64_t D, int dtype, float scale, void* stream) {
  using namespace dg;
  if (!Q || !K || !V || !O) return GEMM_ERR_INVALID_ARG;
  if (BH <= 0 || Sq <= 0 || Sk <= 0 || D <= 0) return GEMM_ERR_INVALID_ARG;
  if (dtype < 0 || dtype > 4 || !std::isfinite(scale)) return GEMM_ERR_INVALID_ARG;
  if (dtype != DT_F16 && dtype != DT_BF16) return GEMM_ERR_UNSUPPORTED;
  if (D != 128) return GEMM_ERR_UNSUPPORTED;
  // every tensor below 2 GiB - 16 (32-bit buffer offsets): with each extent below 2^31 the
  // row counts cannot overflow, and rows * D * 2 >= lim exactly when rows >= row_lim
  const int64_t lim = ((int64_t)1 << 31) - 16;
  if (BH >= lim || Sq >= lim || Sk >= lim) return GEMM_ERR_UNSUPPORTED;
  const int64_t row_lim = (lim + 2 * D - 1) / (2 * D);
  if (BH * Sq >= row_lim || BH * Sk >= row_lim) return GEMM_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return GEMM_ERR_MISALIGNED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_ERR_NO_DEVICE;
  const AttnLaunch l{Q, K, V, O, BH, Sq, Sk, D, dtype, scale};
  const int e = launch_attn(l, stream);
  if (e != 0) {
    if (debug_on()) std::fprintf(stderr, "[dgemm] attention launch failed: %s\n", hipGetErrorString((hipError_t)e));
    return GEMM_ERR_HIP;
  }
  return GEMM_OK;
}

int gemm_lds_row_perm(int block, int stride, int index, int inverse) {
  const dg::RowPerm rp{block, stride};
  if (!rp.valid() || index < 0 || index >= block) return -1;
  return inverse ? rp.inv(index) : rp.fwd(index);
}

}  // extern "C"
