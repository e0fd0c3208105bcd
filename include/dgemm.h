/*
 * dgemm.h -- C ABI of the MI355X (gfx950) operand-layout GEMM library (libdgemm.so).
 *
 * The library computes C = A * B on one GPU, where the logical A is M x K, the logical B
 * is K x N and either operand may be stored row- or column-major. An operand whose K
 * index is not the contiguous one (a "non-TN" operand: Triton PR 5223, "Feature
 * description", where such operands are called K-major / non-KContig) is read with
 * 128-bit coalesced loads, transposed in registers and stored K-contiguous in LDS, so
 * the matrix-core loop reads K-contiguous fragments (when both operands are transposed,
 * they instead stay in global order in LDS and the LDS reads transpose them; see
 * gemm_plan). Skinny shapes split K
 * (BitBLAS PR 268, "SplitK Infer") and reduce the partial sums first across the
 * wavefronts of a workgroup through LDS (IREE PR 19596, inter-subgroup reduction
 * description), then across workgroups. B may instead be 4-bit weight codes with
 * per-group binary16 scales that the loader dequantises (BitBLAS PR 268, dequantize
 * layout example).
 *
 * Conventions for every entry point:
 *   - Return value 0 (GEMM_OK) on success, a negative GEMM_ERR_* code otherwise.
 *   - No entry point aborts, throws across the ABI, prints (unless the environment
 *     variable DGEMM_DEBUG is set) or synchronises the device.
 *   - All argument checks happen before any GPU work is enqueued.
 *   - The library never allocates or frees device memory; the caller owns every device
 *     buffer. The only library-owned object is the host-side plan.
 */
#ifndef DGEMM_H
#define DGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage order of a logical matrix (A is M x K, B is K x N). Row-major: element (r, c)
 * at r * cols + c. Column-major: element (r, c) at r + c * rows. Storage is packed (no
 * leading dimension).
 * GEMM_U4_TILED (int4 B only) is the pre-tiled weight layout of BitBLAS PR 268 (its
 * tiled/"ladder" weight transform): the 64 code bytes of column n and K group g (the
 * 128 codes k = 128g .. 128g+127, low nibble = even k) are stored at byte
 * ((n / 64) * (K / 128) + g) * 4096 + (n % 64) * 64, so every 64 columns x 128 K block is
 * one contiguous 4 KiB run and a workgroup's share of B is one contiguous range.
 * gemm_pack_u4_tiled() converts from the column-major packing. Needs N % 64 == 0. */
enum { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1, GEMM_U4_TILED = 2 };

/* Element types. GEMM_U4 is valid for B only: two 4-bit codes per byte along K.
 * GEMM_F8 is the 8-bit OCP E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * no infinities; S.1111.111 is NaN; largest finite magnitude 448), valid for A and B
 * together, one byte per element. */
enum { GEMM_F32 = 0, GEMM_F16 = 1, GEMM_BF16 = 2, GEMM_U4 = 3, GEMM_F8 = 4 };

/* Status codes. */
enum {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_ARG = -1,         /* null pointer, bad enum, non-positive size */
  GEMM_ERR_UNSUPPORTED = -2,         /* valid request this library does not implement */
  GEMM_ERR_MISALIGNED = -3,          /* a device pointer is not 16-byte aligned */
  GEMM_ERR_WORKSPACE_TOO_SMALL = -4, /* ws_bytes below gemm_workspace_size() */
  GEMM_ERR_NO_DEVICE = -5,           /* no usable HIP device / wrong device current */
  GEMM_ERR_HIP = -6                  /* a HIP runtime call or kernel launch failed */
};

/* Quantisation of an int4 B operand (BitBLAS PR 268, dequantize layout example:
 * num_elems_per_byte = 2). Weight w(k, n) = round_fp16((q(k, n) - zero_point) * s).
 * q(k, n) is the low nibble of byte n*(K/2) + k/2 for even k, the high nibble for odd k.
 * s = scales[(k / group_size) * N + n], binary16 (K / group_size rows of N scales).
 * Supported: group_size a power of two from 32 to K that divides K, zero_point 0..15,
 * scale_dtype = GEMM_F16 and scale_layout = 0 ([K/group][N] row-major). */
typedef struct {
  int32_t group_size;
  int32_t zero_point;
  int32_t scale_dtype;
  int32_t scale_layout;
} gemm_quant_t;

/* Opaque host-side plan. Immutable once made; usable from several streams at once if
 * each concurrent run has its own workspace. */
typedef struct gemm_plan_s* gemm_plan_t;

/* What the planner chose (for reports and tests). */
typedef struct {
  int64_t M, N, K;
  int32_t layout_a, layout_b, dtype_a, dtype_b, dtype_c;
  int32_t kernel;          /* 0 = tiled kernel, 1 = skinny split-K kernel */
  int32_t tile_m, tile_n, tile_k; /* macro tile; tile_k = K elements per main-loop step */
  int32_t waves;           /* wavefronts (64 lanes) per workgroup */
  int32_t lds_pad_bytes;   /* padding after each K-contiguous LDS row of an operand stored by
                              the threads (16; 32 with mfma_m = 16, whose transposed rows also
                              keep 16-byte chunk c of row r at position c ^ ((r >> 2) & 1)) */
  int32_t perm_block;      /* rows per block of the LDS row permutation (1 = none) */
  int32_t perm_stride;     /* stride S of that permutation (rocm-libraries PR 2487) */
  int32_t split_k;         /* K splits across workgroups */
  int32_t wave_split_k;    /* K splits across the waves of one workgroup (1 = none) */
  int64_t grid_x, grid_y, grid_z;
  int64_t workspace_bytes; /* what gemm_run needs (0 when split_k == 1) */
  int32_t lds_bytes;       /* LDS per workgroup */
  int32_t cu_count;        /* compute units of the device */
  int32_t slots_per_cu;    /* resident workgroups per CU the split-K search assumed */
  int32_t direct_lds;      /* bit 0 (A), bit 1 (B): the K-contiguous operand is loaded
                              straight from global memory into LDS (rows of 128 B without
                              padding, 16-byte chunks permuted by an XOR of the row);
                              lds_pad_bytes then applies to the other operand only.
                              bit 2 (A), bit 3 (B): the transposed operand is also loaded
                              straight into LDS in global order (1 KiB blocks plus
                              lds_pad_bytes = 64) and transposed by the LDS reads; on
                              256-wide tiles a block holds two K rows, K rows permuted with
                              perm_block = 8, perm_stride = 4; on other widths (192, 320) a
                              block holds eight 64-wide K-row segments, K rows permuted with
                              perm_block = 64, perm_stride = 8 */
  int32_t schedule;        /* tiled kernel's main loop: 0 = one software pipeline for all
                              waves, 1 = two wave groups in ping-pong (one multiplies while
                              the other reads LDS), 2 = four waves with every operand loaded
                              straight into LDS and one barrier per step (no split-K); 0 for
                              the skinny kernel */
  int32_t mfma_m;          /* rows (= columns) of the matrix-core instruction's output block:
                              32 (v_mfma_f32_32x32x16, fp8 v_mfma_f32_32x32x64) or 16
                              (v_mfma_f32_16x16x32: the skinny kernel, and 8-wave tiles whose
                              per-wave share is not whole 32x32 blocks, e.g. 96x80 of 192x320) */
} gemm_plan_info_t;

/* Make a plan for C (M x N, row-major, dtype_c) = A (M x K) * B (K x N).
 *
 * layout_a/layout_b: GEMM_ROW_MAJOR or GEMM_COL_MAJOR storage of the logical operands.
 * dtype_a: GEMM_F16, GEMM_BF16 or GEMM_F8. dtype_b: the same as dtype_a, or GEMM_U4 with
 *   dtype_a == GEMM_F16, layout_b == GEMM_COL_MAJOR (codes packed along K) or
 *   GEMM_U4_TILED, and a non-null `quant` (otherwise quant must be NULL or is ignored).
 *   fp8 operands are multiplied exactly and summed in fp32 by the matrix cores
 *   (v_mfma_f32_32x32x64_f8f6f4, no block scales) on 256x256 tiles with a K step of 128;
 *   a transposed fp8 operand is transposed in registers at byte granularity and its LDS
 *   rows are permuted with perm_block = 256, perm_stride = 16.
 * dtype_c: GEMM_F32, GEMM_F16 or GEMM_BF16 (round-to-nearest-even from fp32 sums).
 * split_k: 0 lets the planner choose (waste-ratio search over the workgroup slots,
 *   i.e. CU count times resident workgroups per CU, BitBLAS PR 268 "SplitK Infer",
 *   capped at 16); otherwise 1, 2, 4, 8 or 16. A factor above 1 becomes 1 when the output
 *   has more than 16384 tiles (the capacity of the workspace's arrival counters);
 *   gemm_plan_query reports the factor in use.
 * Constraints: M, N, K >= 1; the contiguous extent of each operand is a multiple of 16
 *   bytes, i.e. 8 16-bit or 16 fp8 elements (K for row-major A and column-major B, M for
 *   column-major A, N for row-major B); int4 needs K % 128 == 0. Violations give
 *   GEMM_ERR_UNSUPPORTED.
 * The plan binds to the HIP device current at this call (its CU count feeds the
 * split-K search; the environment variable DGEMM_FAKE_CU_COUNT replaces the query so
 * that planning works without a device). Host only: no allocation, no launch.
 * Loader for a transposed operand: for a column-major A with a column-major B (BLAS NN)
 * and for fp8 it is transposed in registers with byte permutes and stored K-contiguous
 * (Triton PR 5223). For a 16-bit row-major B (BLAS TT and NT) the default is the other
 * loader of the pages (rocm-libraries PR 2487): each transposed operand goes straight into
 * LDS in global order and is transposed by the LDS reads (ds_read_b64_tr_b16), as are
 * NN's A on the non-power-of-2 192x320 tiles (chosen where they fill the CUs). In the
 * environment, DGEMM_FORCE_DTL=2 selects the second loader for any layout (256x256 tiles),
 * DGEMM_FORCE_DTL=0 the in-register transpose of every transposed operand, and
 * DGEMM_FORCE_DTL=1 with DGEMM_FORCE_MFMA=16 the in-register transpose beside a
 * K-contiguous operand loaded straight into LDS; gemm_plan_info_t.direct_lds reports which
 * was chosen.
 * On error *out is set to NULL. */
int gemm_plan(gemm_plan_t* out, int64_t M, int64_t N, int64_t K, int layout_a, int layout_b,
              int dtype_a, int dtype_b, int dtype_c, int split_k, const gemm_quant_t* quant);

/* Host-side repack of int4 codes from the column-major packing (byte n*(K/2) + k/2) into
 * GEMM_U4_TILED (BitBLAS PR 268, tiled weight transform): `codes` and `tiled` are host
 * buffers of N*K/2 bytes each, not overlapping; the scales keep their [K/128][N] layout.
 * Needs N % 64 == 0 and K % 128 == 0 (GEMM_ERR_UNSUPPORTED otherwise), non-null pointers
 * and positive sizes (GEMM_ERR_INVALID_ARG). */
int gemm_pack_u4_tiled(const void* codes, void* tiled, int64_t N, int64_t K);

/* Bytes of device workspace gemm_run needs for this plan (0 when split_k == 1): 64 KiB of
 * arrival counters, then one fp32 partial tile per output tile and K split. The workspace
 * exists because of split-K (BitBLAS PR 268, "SplitK Infer": the K extent is divided among
 * split_k workgroups per output tile, whose partial sums must then be added): the partials
 * left after the cross-wave reduction inside each workgroup (IREE PR 19596, the
 * inter-subgroup reduction description) are added across workgroups through this memory.
 * Host only. Errors: GEMM_ERR_INVALID_ARG for a NULL plan or NULL `bytes`. */
int gemm_workspace_size(gemm_plan_t plan, size_t* bytes);

/* Enqueue C = A * B on `stream` (a hipStream_t; NULL is the default stream) and return
 * without synchronising. The operation is the plain product C(i, j) = sum_k A(i, k) B(k, j)
 * with fp32 sums and one rounding to dtype_c, for operands whose K index need not be the
 * contiguous one (Triton PR 5223, "Feature description"). With split_k > 1 the K extent is
 * divided among split_k workgroups per output tile (BitBLAS PR 268, "SplitK Infer"); inside a
 * workgroup the waves' partial sums are first reduced through LDS (IREE PR 19596, the
 * inter-subgroup reduction description), then across the workgroups through `workspace`. For
 * int4 B the loader dequantises each weight as in gemm_quant_t (BitBLAS PR 268, dequantize
 * layout example).
 * A, B, C (and scales for int4 B) are device pointers in the plan's layouts, each
 * 16-byte aligned; C must not alias A, B or scales. workspace (16-byte aligned,
 * ws_bytes >= gemm_workspace_size) is needed when split_k > 1, else may be NULL.
 * Workspace contract: its first 64 KiB hold arrival counters that must be zero before
 * the workspace is first used; every run that completes leaves them zero again, so a
 * workspace zeroed once can be reused by any plan. Runs that share a workspace must
 * not overlap in time. The rest of the workspace is scratch.
 * Summation order is fixed (split partial sums are added in ascending split index), so
 * repeated runs give identical bits.
 * Ownership: every pointer is the caller's; nothing is retained after the call returns.
 * Errors (returned before anything is enqueued): GEMM_ERR_INVALID_ARG for a NULL plan, A,
 * B, C, scales (int4) or workspace (split_k > 1); GEMM_ERR_MISALIGNED for a pointer that is
 * not 16-byte aligned; GEMM_ERR_WORKSPACE_TOO_SMALL; GEMM_ERR_NO_DEVICE when the current
 * HIP device is not the plan's; GEMM_ERR_HIP when the launch fails. Faults of the kernels
 * themselves surface at the caller's next synchronisation. */
int gemm_run(gemm_plan_t plan, const void* A, const void* B, const void* scales, void* C,
             void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the per-GPU workspace that gemm_run_noalloc uses in place of a caller buffer. */
#define GEMM_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)

/* gemm_run for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same operation, arguments, layouts
 * and results (bit for bit) as gemm_run, without the workspace arguments: a split-K plan
 * uses a workspace of GEMM_NOALLOC_WORKSPACE_BYTES that the library holds in device memory
 * of its own on each GPU it runs on (a static device array, reserved when the library's code
 * is loaded on that GPU and held until the process ends). The first call on a GPU clears the
 * arrival counters at its start with a small kernel on `stream`; every completed run leaves
 * them zero again. No call allocates or frees memory.
 * Calls on the same GPU share that one workspace: calls that overlap in time on one GPU
 * (different streams, or different host threads) race and give wrong results; serialise them.
 * Errors: as gemm_run, plus GEMM_ERR_WORKSPACE_TOO_SMALL when gemm_workspace_size exceeds
 * GEMM_NOALLOC_WORKSPACE_BYTES, and GEMM_ERR_HIP when the device array cannot be resolved. */
int gemm_run_noalloc(gemm_plan_t plan, const void* A, const void* B, const void* scales, void* C,
                     void* stream);

/* Copy the planner's choices into *info: the macro tile, the LDS padding and row
 * permutation of the operand tiles (rocm-libraries PR 2487, "Add support for permuting
 * perpDim" and LdsBlockSizePerPad under "Add support for m0 padding when using LDSTr+DTL"),
 * and the split-K factor (BitBLAS PR 268, "SplitK Infer"). Host only. Errors:
 * GEMM_ERR_INVALID_ARG for a NULL plan or NULL `info`. */
int gemm_plan_query(gemm_plan_t plan, gemm_plan_info_t* info);

/* Free a host plan made by gemm_plan (NULL is ignored). Bookkeeping of this library, not an
 * operation of the pages. The plan must not be in use by a gemm_run call still being made
 * on another host thread; runs already enqueued do not reference it. */
void gemm_plan_destroy(gemm_plan_t plan);

/* Static text for a status code (never NULL; unknown codes give "unknown status").
 * Bookkeeping of this library, not an operation of the pages. */
const char* gemm_status_string(int status);

/* Row permutation used inside LDS tiles (rocm-libraries PR 2487, "Add support for
 * permuting perpDim"): with S' = B / S, forward I' = S*(I mod S') + I / S' and inverse
 * I = S'*(I' mod S) + I' / S. Returns the image of `index` (0 <= index < block) under the
 * forward map (inverse != 0: the inverse map), or -1 when S does not divide B or an
 * argument is out of range. Host-side view of the same function the kernels use. */
int gemm_lds_row_perm(int block, int stride, int index, int inverse);

#ifdef __cplusplus
}
#endif

#endif /* DGEMM_H */
