#pragma once
// HIP kernels for gfx950 (CDNA4): C = A * B with operands in any row/column-major
// layout, fp16/bf16 (or int4 B, or fp8 E4M3 A and B) in, fp32 accumulate, fp32/fp16/bf16
// out.
//
// Tiled kernel, per workgroup and per K step of 128 bytes per row (64 16-bit or 128 fp8 K
// indices):
//   1. 128-bit buffer loads. An operand whose contiguous index is M or N (transposed) is read
//      with consecutive lanes on consecutive 16-byte vectors along that index, each lane
//      taking four consecutive K rows of its vector (the "thread rake" of Triton PR 5223,
//      item 2), so every load instruction covers whole 128-byte lines. A K-contiguous operand
//      is read as whole 128-byte row segments, by default straight into LDS
//      (buffer_load ... lds, no registers, XOR-swizzled 16-byte chunks).
//   2. In-register transpose of each lane's 4 x 8 block of 16-bit values (4 x 16 bytes for
//      fp8) with byte permutes (v_perm_b32; Triton PR 5223, "Feature description"), giving
//      K-contiguous pieces per M/N index.
//   3. LDS stores into padded, row-permuted, K-contiguous tiles (lds_layout.hpp).
//   4. 128-bit LDS reads of matrix-core fragments, v_mfma_f32_32x32x16_{f16,bf16} or
//      v_mfma_f32_32x32x64_f8f6f4. Two LDS stages, register loads two steps ahead,
//      direct-to-LDS loads one step ahead. Main loop: two wave groups in ping-pong (one
//      multiplies while the other reads LDS, stores and loads; a fenced barrier after every
//      phase), or a software pipeline with one barrier per step. A transposed 16-bit operand
//      can also go straight into LDS in global order and be transposed by ds_read_b64_tr_b16
//      (rocm-libraries PR 2487's direct-to-LDS layout with padding and row permutation); the
//      planner takes that loader when both operands are transposed.
//   5. Split-K across workgroups (BitBLAS PR 268, "SplitK Infer"; the K origin of split
//      z is z * k_chunk): each split stores its fp32 partial tile; the last split to
//      arrive at the tile's counter adds all partials in ascending split order.
//   6. Epilogue: fp32 -> output type (round to nearest even), staged through LDS so
//      that global stores are whole 16-byte row vectors.
//
// Skinny kernel (M <= 16, K-contiguous A and B, or int4 B): every wave of a workgroup
// owns an interleaved share of the workgroup's K range and loads matrix-core fragments
// straight from HBM; the waves' partial tiles are then reduced through LDS
// (IREE PR 19596: partial reductions left across subgroups are re-distributed through
// shared memory into element tiles and reduced again), then across workgroups as above.
//
// int4 B: 4-bit codes packed two per byte along K, (q - z) * s rounded once to binary16, one
// scale per group of K indices (BitBLAS PR 268, dequantize layout example with
// num_elems_per_byte = 2; zero point z and group size are plan parameters).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lds_layout.hpp"
#include "plan.hpp"

namespace dg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer offset beyond every operand's num_records: such a load returns zeros.
constexpr uint32_t kOOB = 0x80000000u;

// Over-synchronised build (compiled with -DDGEMM_OVERSYNC=1 into a separate test library):
// in the tiled kernel's main loops every phase ends with a wait for every outstanding load
// and LDS access and a workgroup barrier. It computes the same sums in the same order, so
// its results must equal the normal build's bit for bit; a difference would expose an LDS
// race that the hand-ordered waits and barriers of the normal build leave open.
#ifndef DGEMM_OVERSYNC
#define DGEMM_OVERSYNC 0
#endif
constexpr bool kOverSync = DGEMM_OVERSYNC != 0;
__device__ __forceinline__ void oversync_point() {
  if constexpr (kOverSync) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct F16T {};
struct BF16T {};
struct F8T {};   // OCP 8-bit E4M3 (bias 7, no infinities, S.1111.111 is NaN)

// Bytes per operand element; every main-loop step moves 128-byte LDS rows, i.e. 64 K
// indices of a 16-bit type or 128 of fp8.
template <class T>
constexpr int elem_bytes() { return std::is_same<T, F8T>::value ? 1 : 2; }

template <class T>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16x16x32<F16T>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16x16x32<BF16T>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // Raw buffer (stride 0); word 3 = 32-bit data format, the gfx9-family default.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t ld16b(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ---------------------------------------------------------------- register transforms

// 8x8 block of 16-bit values: in[kk] holds K row kk, elements e = 0..7 (two per dword,
// element 2d in the low half of dword d). Out[e] holds element e for K rows 0..7 (K row
// 2t in the low half of dword t). v_perm_b32 (D, S0, S1, sel): byte i of D is byte
// sel.byte[i] of the 8-byte value S0:S1 (S1 = bytes 0..3). Selector 0x05040100 joins the
// low halves of S1 and S0, 0x07060302 their high halves.
// Output row e of a 4 x 8 block (four K rows of eight elements): its four K values as
// two dwords (two byte permutes).
__device__ __forceinline__ u32x2 transpose_row4(const u32x4 (&in)[4], int e) {
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  u32x2 r;
  r[0] = __builtin_amdgcn_perm(in[1][e >> 1], in[0][e >> 1], sel);
  r[1] = __builtin_amdgcn_perm(in[3][e >> 1], in[2][e >> 1], sel);
  return r;
}

// 4x4 block of bytes (fp8 values): r0..r3 are K rows 0..3, byte e of each holds element
// e along M/N. Out o[e] holds element e for K rows 0..3 (byte j = K row j). The same byte
// permute transpose as for 16-bit values, at byte granularity: the first pair of permutes
// interleaves the bytes of rows (0, 1) and (2, 3), the second joins the 16-bit halves.
__device__ __forceinline__ void transpose_bytes4(uint32_t r0, uint32_t r1, uint32_t r2,
                                                 uint32_t r3, uint32_t (&o)[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
  const uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
  const uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Eight 4-bit codes of one dword (byte b: low nibble = code of K index 2b, high nibble =
// code of 2b+1) -> eight binary16 weights (q - z) * s, K-consecutive, as four dwords.
// 0x6400 | q is the binary16 encoding of 1024 + q, so subtracting bias = 1024 + z gives
// q - z exactly; the one rounding is the binary16 multiply by s.
__device__ __forceinline__ u32x4 dequant8(uint32_t w, f16x2 s2, f16x2 bias) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  u32x4 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // byte t of lo -> bits 0..7, byte t of hi -> bits 16..23, zeros elsewhere (sel 0x0C).
    const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + t) << 16) | (uint32_t)t;
    const uint32_t q2 = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
    f16x2 v = __builtin_bit_cast(f16x2, q2) - bias;
    v = v * s2;
    r[t] = __builtin_bit_cast(uint32_t, v);
  }
  return r;
}

// The same eight weights for a matrix-core fragment whose K order may be permuted (the
// activation fragment is permuted to match): dword j holds the weights of K indices j and
// j+4 (nibbles j and j+4). Each pair comes out of one and-or as binary16 values: a nibble
// in bits 0..3 of a half gives 0x6400 | q = 1024 + q, one in bits 4..7 gives 1024 + 16q.
// (1024 + q) - (1024 + z) and (1024 + 16q) / 16 - (64 + z) are q - z exactly (one fused
// multiply-add, exact because the result is representable); the multiply by s is the single
// rounding. bias = -(1024 + z), bias16 = -(64 + z).
// 13 instructions per eight weights instead of 19.
// (x & mask) | magic in one instruction (the compiler splits it into two with literals).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
  return r;
}

__device__ __forceinline__ u32x4 dequant8_pairs(uint32_t w, f16x2 s2, f16x2 bias, f16x2 bias16) {
  const uint32_t w8 = w >> 8;
  const uint32_t magic = 0x64006400u;
  const uint32_t t0 = and_or(w, 0x000F000Fu, magic);    // nibbles 0, 4
  const uint32_t t1 = and_or(w, 0x00F000F0u, magic);    // nibbles 1, 5 (times 16)
  const uint32_t t2 = and_or(w8, 0x000F000Fu, magic);   // nibbles 2, 6
  const uint32_t t3 = and_or(w8, 0x00F000F0u, magic);   // nibbles 3, 7 (times 16)
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, t0) + bias) * s2);
  r[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, t1), sixteenth, bias16) * s2);
  r[2] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, t2) + bias) * s2);
  r[3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, t3), sixteenth, bias16) * s2);
  return r;
}

// Eight consecutive 16-bit values (K indices 0..7, two per dword) reordered to the K order
// of dequant8_pairs: dword j = (value j, value j + 4).
__device__ __forceinline__ u32x4 pair_k_and_k4(u32x4 d) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
  return r;
}

// ---------------------------------------------------------------- output conversion

template <int DT> struct OutT;
template <> struct OutT<DT_F32> { using type = float; static constexpr int bytes = 4; };
template <> struct OutT<DT_F16> { using type = _Float16; static constexpr int bytes = 2; };
template <> struct OutT<DT_BF16> { using type = __bf16; static constexpr int bytes = 2; };

template <int DT>
__device__ __forceinline__ typename OutT<DT>::type cvt_out(float x) {
  return (typename OutT<DT>::type)x;  // round to nearest even
}

// ---------------------------------------------------------------- kernel arguments

struct KArgs {
  const void* A;
  const void* B;
  const void* S;        // int4 scales (binary16, [K/group][N])
  void* C;
  float* part;          // fp32 partials (split-K), after the counters
  int* counters;        // arrival counters (split-K)
  int M, N, K;
  int ldA, ldB;         // leading dimension of the stored operands
  uint32_t bytesA, bytesB, bytesS;
  int k_chunk;          // K per split (multiple of the K step)
  int tiles_m, tiles_n;
  int dtype_c;
  int c_vec;            // 1 if every C row starts 16-byte aligned
  int b_tiled;          // int4 codes in the pre-tiled layout (64 columns x 128 K blocks)
  int group_log2;       // int4: log2 of the scale group size (5 .. log2 K)
  int zero;             // int4: zero point (0 .. 15)
};

// Split-K fix-up shared by both kernels. Threads tid < LIVE own NV vectors of LEN fp32
// partial sums (the others own nothing: the skinny kernel's reduced tile has fewer
// positions than threads); the workgroup stores them into split z's slot, the last
// workgroup to arrive at the tile's counter adds all splits in ascending split order and
// returns true; the others return false. The counter is reset for the next run.
//
// Cross-XCD visibility without cache maintenance: partials are written and read with
// agent-scope relaxed atomics (device-coherent stores and loads that go to the memory
// side, past the XCD-private L2), every thread waits for its stores to complete before
// the workgroup barrier, and only then is the counter incremented (agent scope). An
// agent-scope release/acquire fence would instead write back and invalidate the whole
// L2 of the XCD for every workgroup. Layout: element-major [split][tile][v][e][live thread],
// so every store and load instruction covers consecutive addresses.
template <class V, int NV, int THREADS, int LIVE = THREADS>
__device__ __forceinline__ bool splitk_fixup(V (&acc)[NV], const KArgs& a, int tile,
                                             int z, int sk, int tiles) {
  constexpr int LEN = sizeof(V) / sizeof(float);
  static_assert(LIVE <= THREADS && (NV == 1 || LIVE == THREADS), "live threads");
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const bool live = tid < LIVE;
  const size_t per_tile = (size_t)NV * LEN * LIVE;
  float* mine = a.part + ((size_t)z * tiles + tile) * per_tile;
  if (live) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < LEN; ++e)
        __hip_atomic_store(mine + ((size_t)v * LEN + e) * LIVE + tid, acc[v][e], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(a.counters + tile, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == sk - 1);
  }
  __syncthreads();
  if (!s_last) return false;
  const float* base = a.part + (size_t)tile * per_tile;
  const size_t split_stride = (size_t)tiles * per_tile;
  if (live) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
#pragma unroll
      for (int e = 0; e < LEN; ++e) {
        const size_t idx = ((size_t)v * LEN + e) * LIVE + tid;
        float s = (z == 0) ? acc[v][e] : __hip_atomic_load(base + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int b = 1; b < sk; ++b)
          s += (b == z) ? acc[v][e]
                        : __hip_atomic_load(base + b * split_stride + idx, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        acc[v][e] = s;
      }
    }
  }
  if (tid == 0)
    __hip_atomic_store(a.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// ================================================================= tiled kernel

// One load slot of a thread: a block of VPB 16-byte vectors of one operand per K step.
template <int VPB>
struct Slot {
  uint32_t off[VPB];  // byte offsets at the split's first K step (kOOB when outside)
  int kofs;           // K index, relative to the step start, of the block's first element
  int wbase;          // LDS byte offset of the block's first store (stage-relative)
  int row;            // int4: N index of the block's row (scale lookup)
};

// How a thread moves its share of one operand tile (ROWS M or N indices x one K step of
// 128 bytes per row: BK = 64 16-bit or 128 fp8 K indices) from HBM to LDS. KIND 0:
// K-contiguous storage. KIND 1: 16-bit values contiguous along M/N (the operand is
// transposed in registers). KIND 2: int4 codes packed along K. KIND 3: fp8 values
// contiguous along M/N (transposed in registers at byte granularity).
//   KIND 0, block q, vector j: row j*ROWS/4 + q/8, 16-byte chunk q%8 of the step. Eight
//     consecutive lanes cover one 128-byte row segment: whole lines in HBM, one LDS row.
//   KIND 1, block q: kh = q%2, v = (q/2) % (ROWS/8), kg = (q/2) / (ROWS/8); vector j is K
//     row 8kg + 4kh + j of elements 8v..8v+7 (thread rake: four consecutive K rows of one
//     16-byte vector along M/N); consecutive lanes cover consecutive vectors of a K row.
//     After the byte-permute transpose, element e's four K values (8 bytes) go to LDS
//     row inv(8v + e) at byte 16kg + 8kh. The 16 lanes of one 64-bit store phase hold
//     eight consecutive v and both kh: with the 64-row, stride-8 permutation they hit
//     eight consecutive LDS rows (eight 16-byte bank groups) times two 8-byte halves.
//   KIND 2, block q: row q/2, K half q%2 (32 codes, 16 bytes) -> four 16-byte stores of
//     eight binary16 weights each.
//   KIND 3, block q = 32 h + 8 kl + vl (vl < 8, kl < 4): v = vl + 8 (h % (ROWS/128)),
//     kg = kl + 4 (h / (ROWS/128)); vector j is K row 4kg + j of elements 16v..16v+15 (eight
//     consecutive lanes read one 128-byte line). After the byte transpose, element e's four K
//     values (one dword) go to LDS row inv(16v + e) at byte 4kg. With the 256-row, stride-16
//     permutation, inv(16v + e) = 16e + v, and a row's dword offset is 36 row: the 32 lanes
//     of one 128-byte store phase (eight v, four kg) hit dwords 36 v + kg, all different
//     modulo 32 (and the 64 lanes of the wave all different modulo 64).
// PITCH 160 (the 16x16x32 kernels' transposed operands): 32 bytes of padding, and in every
// LDS row r the 16-byte chunk c is kept at position c ^ ((r >> 2) & 1). Measured with the
// bank-conflict counter on gfx950: at the 144-byte pitch the 16-row fragment reads of a
// 16x16x32 block (16 rows x four chunks per instruction) take two passes, at 160 bytes the
// transposing stores do, and at 160 bytes with this chunk swap neither does (the 32-row
// reads of 32x32x16 blocks are conflict-free at 144 bytes, which those kernels keep).
template <int KIND, int ROWS, int THREADS, RowPerm P, int EB = 2, int PITCH = 144>
struct Operand {
  static constexpr int BK = 128 / EB;
  // LDS row pitch: 128 B of data plus 16 B (or 32 B) of padding (128: no padding, a
  // comparison variant whose fragment reads and transposed stores meet bank conflicts)
  static constexpr int PITCH_B = PITCH;
  static constexpr bool CSWZ = PITCH == 160;   // chunk c of row r at c ^ ((r >> 2) & 1)
  static constexpr int VPB = KIND == 2 ? 1 : 4;
  static constexpr int BLOCKS = ROWS * 2;            // blocks per K step
  static constexpr int SLOTS = (BLOCKS + THREADS - 1) / THREADS;
  static constexpr bool PARTIAL = BLOCKS % THREADS != 0;
  // Elements per 16-byte vector along M/N of a transposed operand.
  static constexpr int VL = KIND == 3 ? 16 : 8;
  // LDS-row step between the rows of one transposed vector: inv(VL*v + e) = inv(VL*v) + e*ES.
  static constexpr int ES = P.block == 1 ? 1 : P.block / P.stride;
  static constexpr bool es_ok() {
    for (int v = 0; v < ROWS / VL; ++v)
      for (int e = 0; e < VL; ++e)
        if (P.inv(VL * v + e) != P.inv(VL * v) + e * ES) return false;
    return true;
  }
  static_assert(es_ok(), "row permutation must step evenly inside a vector");
  static_assert(!CSWZ || ES % 8 == 0, "chunk swap: a block's eight rows must share bit 2");
  static_assert(ROWS % 64 == 0 && ROWS % P.block == 0, "tile rows must be whole permutation blocks");
  static_assert((KIND != 1 && KIND != 2) || EB == 2, "16-bit operand kinds");
  static_assert(KIND != 3 || EB == 1, "fp8 operand kind");
  static_assert(!(PARTIAL && KIND == 2), "int4 blocks must fill every thread");
  static_assert(PITCH == 144 || (PITCH == 128 && !PARTIAL && KIND != 2) || (PITCH == 160 && KIND == 1),
                "unpadded rows: no idle lanes (they store into the padding), no int4; the chunk "
                "swap of 160-byte rows: transposed 16-bit operands only");

  // Block q of this K split: offsets, K offset and LDS base. Blocks past BLOCKS (idle
  // lanes of a partial slot) read nothing (zeros) and store them into padding bytes of
  // their own tile: byte 128 of a row is its pad, and every store offset of a block is a
  // multiple of the row pitch plus at most the pad's 16 bytes.
  __device__ __forceinline__ static void setup(Slot<VPB>& s, int q, int row0, int rows_total,
                                               int ld, int kb, int K, bool tiled = false) {
    const bool live = q < BLOCKS;
    if constexpr (KIND == 0) {
      const int c = q % 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = j * (ROWS / 4) + q / 8;
        s.off[j] = (live && row0 + r < rows_total) ? (uint32_t)((row0 + r) * ld + kb) * EB + 16u * c : kOOB;
      }
      s.kofs = 16 * c / EB;
      s.wbase = P.inv(q / 8) * PITCH_B + 16 * c;
    } else if constexpr (KIND == 1) {
      const int kh = q % 2, v = (q / 2) % (ROWS / 8), kg = (q / 2) / (ROWS / 8);
      const bool ok = live && row0 + 8 * v < rows_total;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s.off[j] = ok ? (uint32_t)((kb + 8 * kg + 4 * kh + j) * ld + row0 + 8 * v) * 2u : kOOB;
      s.kofs = 8 * kg + 4 * kh;
      // rows inv(8v) + e*ES (ES a multiple of 8) share bit 2, so one chunk position serves
      // all eight stores of the block
      const int r0 = P.inv(8 * v);
      s.wbase = r0 * PITCH_B + 16 * (CSWZ ? (kg ^ ((r0 >> 2) & 1)) : kg) + 8 * kh;
    } else if constexpr (KIND == 3) {
      static_assert(ROWS % 128 == 0, "eight 16-byte vectors per store phase");
      const int h = q >> 5;
      const int v = (q & 7) + 8 * (h % (ROWS / 128)), kg = ((q >> 3) & 3) + 4 * (h / (ROWS / 128));
      const bool ok = live && row0 + 16 * v < rows_total;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s.off[j] = ok ? (uint32_t)((kb + 4 * kg + j) * ld + row0 + 16 * v) : kOOB;
      s.kofs = 4 * kg;
      s.wbase = P.inv(16 * v) * PITCH_B + 4 * kg;
    } else {
      const int r = q / 2, h = q % 2;
      // column-major packing: byte n*(K/2) + k/2; pre-tiled: 4 KiB blocks of 64 columns x
      // 128 K, 64 bytes per column (the split start kb is a multiple of 128)
      const int n = row0 + r;
      const uint32_t o = tiled ? ((uint32_t)((n / 64) * (K / 128) + kb / 128) * 64u + (uint32_t)(n % 64)) * 64u + 16u * h
                               : (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)((kb + 32 * h) / 2);
      s.off[0] = (live && n < rows_total) ? o : kOOB;
      s.kofs = 32 * h;
      s.wbase = P.inv(r) * PITCH_B + 64 * h;
      s.row = row0 + r;
    }
    if (!live) s.wbase = 128;  // row 0's pad (KIND 0: rows j*ROWS/4, KIND 1/3: rows e*ES)
  }
};

// A K-contiguous operand moved by direct global->LDS loads (buffer_load ... lds): the
// data never passes through registers and no LDS store instruction is issued, so the
// wave keeps issuing matrix-core instructions while the tile streams in. LDS rows are
// 128 bytes (64 K values) without padding; the 16-byte chunk c of row r is kept in slot
// c ^ swz(r), swz(r) = (r >> 1) & 7 (a chunk permutation of the K-contiguous layout), so
// that a fragment read (lanes on 32 consecutive rows, one chunk each) touches every bank
// group once per 16 lanes (the row is 64 16-bit or 128 fp8 K values; the chunks are the
// same 16-byte units). One load instruction of a wave fills eight whole LDS rows
// (1 KiB): lane t writes row t/8, slot t%8, and therefore loads chunk (t%8) ^ swz(row) of
// that row, so the eight lanes of a row still read one whole 128-byte line.
__device__ __forceinline__ constexpr int dtl_swz(int r) { return (r >> 1) & 7; }

// Buffer resource words (base, stride 0, num_records, gfx9-family data format) for
// instructions written as inline assembly.
__device__ __forceinline__ u32x4 rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p);
}

template <int ROWS, int THREADS, int EB = 2>
struct DtlOperand {
  static constexpr int WAVES = THREADS / 64;
  static constexpr int NI = ROWS / (8 * WAVES);  // load instructions per wave and K step
  static_assert(ROWS % (8 * WAVES) == 0, "every wave fills whole groups of eight rows");
  uint32_t off[NI];  // byte offsets at the split's first K step (kOOB outside the operand)
  int kofs[NI];      // K index of the lane's chunk relative to the step start

  __device__ __forceinline__ void setup(int lane, int wave, int row0, int rows_total, int ld,
                                        int kb) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = 8 * (wave * NI + j) + lane / 8;
      const int c = (lane & 7) ^ dtl_swz(r);
      off[j] = row0 + r < rows_total ? (uint32_t)((row0 + r) * ld + kb) * EB + 16u * c : kOOB;
      kofs[j] = 16 * c / EB;
    }
  }
  // Loads of one K step (byte step d from the split's first step; lim = K indices left)
  // into the operand's LDS region at byte address `base` of one stage. Written as inline
  // assembly so that the compiler, which cannot tell the LDS regions apart, does not make
  // every later LDS access wait for these loads; the kernel waits for them itself (a full
  // s_waitcnt before the barrier that ends the step). The wait states cover a scalar
  // register written by a vector instruction just before (the resource and M0 value) and
  // the M0 write before an LDS-bound load.
  __device__ __forceinline__ void issue(const u32x4& rs, uint32_t base, int wave, uint32_t d,
                                        int lim) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) issue_one(rs, base, wave, d, lim, j);
  }
  // Load instruction j of the step only.
  __device__ __forceinline__ void issue_one(const u32x4& rs, uint32_t base, int wave, uint32_t d,
                                            int lim, int j) const {
    const uint32_t o = kofs[j] < lim ? off[j] + d : kOOB;
    const uint32_t m0v = base + (uint32_t)(wave * NI + j) * 1024u;
    asm volatile(
        "s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
        :
        : "v"(o), "s"(m0v), "s"(rs)
        : "memory", "m0");
  }
};

// An operand whose contiguous index is M or N (ROWS of them per tile, a multiple of 64),
// moved by direct global->LDS loads and transposed on the read instead of in registers
// (rocm-libraries PR 2487: direct-to-LDS with padding per LDS block and a permutation of the
// perpendicular dimension, for power-of-2 and other macro tiles alike). Every load
// instruction of a wave fills one 1 KiB LDS block, followed by 64 bytes of padding (the pad
// goes in through the per-instruction LDS base, as the page's m0 padding). Each lane moves
// 16 bytes, so the divisions that map a lane to its K row and M chunk are by powers of 2 for
// any ROWS.
// ds_read_b64_tr_b16 (gfx950) gives lane t of each 16-lane group element t%4 of the 8-byte
// chunks addressed by lanes t/4 + 4e, e = 0..3. Reading, per 16-lane group, K rows
// kb + 4r + s/4 at M chunk s%4 (s = lane%16) gives lane t M index t and the four K values
// kb + 4r .. kb + 4r + 3; two reads (r = 0, 1) make one v_mfma_f32_32x32x16 fragment in
// natural K order. Lanes 32..63 read K rows kb + 8 .. kb + 15.
// Two block layouts, both free of bank conflicts for these reads (the four K rows a
// half-wave reads lie in four consecutive blocks at the same in-block offset, 1088 B apart,
// i.e. at bank offsets 0, 64, 128 and 192 B):
//  - ROWS == 256 (ROWS-wide K rows, 512 B): a block holds two K rows (lane t: row t/32,
//    elements 8(t%32)..+7). Within each group of eight K rows the rows are placed with the
//    page's permutation B = 8, S = 4: LDS row L of the group holds K row 4(L%2) + L/2, so
//    block j holds K rows j and j+4.
//  - other ROWS (192, 320, ...: the non-power-of-2 macro tiles): the tile is cut into
//    64-wide segments and a block holds eight 128-byte K rows of one segment (lane t: row
//    i = t/8, LDS chunk t%8, whole 128-byte lines of global memory). The 64 K rows of a
//    step are placed with the page's permutation B = 64, S = 8: LDS row I = 8b + i (block b
//    of the segment, row i) holds K row 8i + b, so consecutive K rows go to consecutive
//    blocks, i.e. to different load instructions, and the m0 padding separates their banks.
//    In odd rows the 16-byte chunks of a segment are stored with chunk c at position c ^ 2.
//    A 32x32x16 fragment read (two 16-lane groups on the same four rows, 32 M values)
//    never pairs an odd row with an even one; for the 16x16x32 reads (16 M values, the two
//    16-lane groups of a half-wave on rows i and i + 1 of the same four blocks, 128 B
//    apart) the swap moves the odd row's 32 bytes to the other half of the same 64-byte
//    bank group, so both shapes read free of bank conflicts.
template <int ROWS, int THREADS, bool SEG_ = ROWS != 256>
struct DtlTrOperand {
  static_assert(ROWS % 64 == 0, "whole 64-wide segments");
  static constexpr bool SEG = SEG_;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int BLOCKS = ROWS / 8;         // 64 K rows x ROWS x 2 B per step, 1 KiB each
  static constexpr int NI = BLOCKS / WAVES;       // load instructions per wave and K step
  static constexpr int BLOCK_BYTES = 1024 + 64;   // data + padding
  static constexpr int BYTES = BLOCKS * BLOCK_BYTES;
  static constexpr RowPerm P = SEG ? RowPerm{64, 8} : RowPerm{8, 4};
  // Byte distances between the reads of one fragment (r = 1 against r = 0) and between
  // 16-K sub-steps.
  static constexpr int R1 = SEG ? 4 * BLOCK_BYTES : 512;
  static constexpr int KK_BYTES = SEG ? 256 : 8 * BLOCK_BYTES;
  static_assert(BLOCKS % WAVES == 0, "whole blocks per wave");
  uint32_t off[NI];  // byte offsets at the split's first K step (kOOB outside the operand)
  int krow[NI];      // K row of the lane, relative to the step start

  __device__ __forceinline__ void setup(int lane, int wave, int row0, int rows_total, int ld,
                                        int kb) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int b = wave * NI + j;
      int k, m;
      if constexpr (SEG) {   // block b: segment b/8, K rows P.fwd(8(b%8) + i), i = row in block
        const int i = lane / 8;
        k = P.fwd(8 * (b % 8) + i);
        m = row0 + 64 * (b / 8) + 8 * ((lane % 8) ^ (2 * (i & 1)));
      } else {               // block b: group b/4, slot b%4
        k = 8 * (b / 4) + P.fwd(2 * (b % 4) + lane / 32);
        m = row0 + 8 * (lane % 32);
      }
      off[j] = m < rows_total ? (uint32_t)((kb + k) * ld + m) * 2u : kOOB;
      krow[j] = k;
    }
  }
  __device__ __forceinline__ void issue(const u32x4& rs, uint32_t base, int wave, uint32_t d,
                                        int lim) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) issue_one(rs, base, wave, d, lim, j);
  }
  __device__ __forceinline__ void issue_one(const u32x4& rs, uint32_t base, int wave, uint32_t d,
                                            int lim, int j) const {
    const uint32_t o = krow[j] < lim ? off[j] + d : kOOB;
    const uint32_t m0v = base + (uint32_t)(wave * NI + j) * BLOCK_BYTES;
    asm volatile(
        "s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
        :
        : "v"(o), "s"(m0v), "s"(rs)
        : "memory", "m0");
  }
  // LDS byte offset (stage-relative) of M (or N) index m of the K row that is row i of
  // block b of m's segment (segment layout).
  __device__ __forceinline__ static int seg_off(int b, int i, int m) {
    return (8 * (m / 64) + b) * BLOCK_BYTES + i * 128 + ((((m % 64) / 8) ^ (2 * (i & 1))) * 16) +
           (m % 8) * 2;
  }
  // Lane's byte offset (stage-relative) of the 32x32x16 fragment whose 32 M (or N) indices
  // start at col (a multiple of 32), for sub-step 0 and read 0; sub-step kk adds
  // KK_BYTES * kk, read 1 adds R1.
  __device__ __forceinline__ static int frag_off(int lane, int col) {
    const int G = lane / 16, s = lane % 16;
    const int m = col + 16 * (G % 2) + 4 * (s % 4);
    if constexpr (SEG)
      return seg_off(s / 4, G / 2, m);
    else
      return (4 * (G / 2) + s / 4) * BLOCK_BYTES + m * 2;
  }
  // The same for a 16x16x32 fragment (16 M or N indices from col, a multiple of 16; lane
  // group G = lane/16 takes K rows 8G .. 8G + 7 of the 32-K half step): half step h adds
  // KK16_BYTES * h, read 1 adds R1. Segment layout only (in the two-row layout the eight
  // blocks a half-wave reads would meet in pairs on the same banks).
  static constexpr int KK16_BYTES = 4 * 128;
  __device__ __forceinline__ static int frag_off16(int lane, int col) {
    static_assert(SEG, "16x16x32 fragments: segment layout");
    const int G = lane / 16, s = lane % 16;
    return seg_off(s / 4, G, col + 4 * (s % 4));
  }
};

// One v_mfma_f32_32x32x16 fragment from a transposed LDS block: reads at p and p + R1.
template <int R1>
__device__ __forceinline__ u32x4 tr_fragment(const char* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)p);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p + R1));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// LROWS, the LDS rows of operands stored by the threads: 1 = permuted (transposed operands)
// and padded, 0 = identity order and padded, 2 = identity order without padding. 0 and 2
// are comparison variants for bank-conflict measurements.
// MI: the matrix-core block, 32 (v_mfma_f32_32x32x16, fp8 32x32x64) or 16
// (v_mfma_f32_16x16x32; the 8-wave tiles whose wave tiles are not whole 32x32 blocks, e.g.
// 96x80 in 192x320).
template <class T, bool A_KC, bool B_KC, bool U4B, int MT_M, int MT_N, int WM, int WN,
          int LROWS, int DTL, int MI = 32>
struct TileCfg {
  static constexpr int EB = elem_bytes<T>();
  static constexpr bool F8 = EB == 1;
  static constexpr int BK = 128 / EB;                    // K per step: 128-byte LDS rows
  static constexpr int THREADS = WM * WN * 64;
  static constexpr int WT_M = MT_M / WM, WT_N = MT_N / WN;
  static constexpr int TM = WT_M / MI, TN = WT_N / MI;   // MIxMI blocks per wave
  static_assert(MI == 32 || MI == 16, "matrix-core block");
  // Direct-to-LDS loads (DTL >= 1) for K-contiguous operands (not for int4 codes, which
  // are dequantised in registers); with DTL == 2 also for the transposed operands, which
  // are then transposed by the LDS reads instead of in registers.
  static constexpr bool A_DTL = DTL >= 1 && A_KC;
  static constexpr bool B_DTL = DTL >= 1 && B_KC && !U4B;
  static constexpr bool A_TR = DTL == 2 && !A_KC;
  static constexpr bool B_TR = DTL == 2 && !B_KC && !U4B;
  static_assert(!(F8 && (DTL == 2 || U4B)), "fp8: no transposing LDS reads, no int4 B");
  static constexpr bool ANY_DTL = A_DTL || B_DTL || A_TR || B_TR;
  // LDS row permutation of an operand transposed in registers (see Operand).
  static constexpr RowPerm PT = F8 ? RowPerm{256, 16} : RowPerm{64, 8};
  static constexpr RowPerm PA = (!A_KC && LROWS == 1 && !A_TR) ? PT : RowPerm{1, 1};
  static constexpr RowPerm PB = (!B_KC && !U4B && LROWS == 1 && !B_TR) ? PT : RowPerm{1, 1};
  static_assert(LROWS >= 0 && LROWS <= 2 && (LROWS != 2 || (DTL == 0 && !U4B)),
                "unpadded rows: a comparison variant of the register-staged kernels");
  static constexpr int PITCH = LROWS == 2 ? 128 : 144;
  // 16x16x32 blocks read 16 rows per instruction: an operand they take transposed through
  // registers gets 160-byte rows with a chunk swap (Operand)
  static constexpr int PITCH_OA = (MI == 16 && !A_KC && !A_TR && LROWS == 1) ? 160 : PITCH;
  static constexpr int PITCH_OB = (MI == 16 && !B_KC && !B_TR && !U4B && LROWS == 1) ? 160 : PITCH;
  static constexpr bool CSWZ_A = PITCH_OA == 160, CSWZ_B = PITCH_OB == 160;
  static constexpr int KT = F8 ? 3 : 1;                  // kind of a transposed operand
  using OpA = Operand<A_KC ? 0 : KT, MT_M, THREADS, PA, EB, PITCH_OA>;
  using OpB = Operand<U4B ? 2 : (B_KC ? 0 : KT), MT_N, THREADS, PB, EB, PITCH_OB>;
  using DA = DtlOperand<MT_M, THREADS, EB>;
  using DB = DtlOperand<MT_N, THREADS, EB>;
  // (the 16x16x32 kernels read transposed operands from the segment layout at any width)
  using TA = DtlTrOperand<A_TR ? MT_M : 256, THREADS, (A_TR ? MT_M : 256) != 256 || MI == 16>;
  using TB = DtlTrOperand<B_TR ? MT_N : 256, THREADS, (B_TR ? MT_N : 256) != 256 || MI == 16>;
  // Register-staged load slots per thread (none for a direct-to-LDS operand).
  static constexpr int SA = (A_DTL || A_TR) ? 0 : OpA::SLOTS;
  static constexpr int SB = (B_DTL || B_TR) ? 0 : OpB::SLOTS;
  // LDS row pitch in 16-byte units: 128 B of data, plus 16 B of padding for operands
  // stored by the threads (none for direct-to-LDS rows, which use the chunk swizzle).
  static constexpr int PA16 = A_DTL ? 8 : PITCH_OA / 16, PB16 = B_DTL ? 8 : PITCH_OB / 16;
  static constexpr int A16 = A_TR ? TA::BYTES / 16 : MT_M * PA16;
  static constexpr int B16 = B_TR ? TB::BYTES / 16 : MT_N * PB16;
  static constexpr int STAGE16 = A16 + B16;
  static constexpr int LDS_BYTES = 2 * STAGE16 * 16;
  // LDS the kernel allocates (every schedule: the two stages)
  static constexpr int lds_alloc(int) { return LDS_BYTES; }
  // Register sets for in-flight global data: two (loads two steps ahead) unless a thread
  // owns more than four blocks, where the second set would not fit in the register file.
  static constexpr int NSETS = (SA + SB) > 4 ? 1 : 2;
  static_assert(!ANY_DTL || NSETS == 2, "direct-to-LDS schedule keeps loads a step ahead");
  static_assert(WT_M % MI == 0 && WT_N % MI == 0, "wave tile must be whole MIxMI blocks");
  // 16x16x32 blocks: 16-bit operands (fp8 has its own 32x32x64 step; int4 B, whose codes
  // and scales are staged in registers, would spill with accumulators in VGPRs)
  static_assert(MI == 32 || (!F8 && !U4B), "16x16x32 blocks: 16-bit operands");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class T>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32x32x16<F16T>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32x32x16<BF16T>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x64_f8f6f4 with both operands fp8 E4M3 (format code 0) and no block
// scales: a lane's fragment is 32 bytes, given here as two 16-byte halves.
__device__ __forceinline__ f32x16 mfma32x32x64_f8(const u32x4 (&a)[2], const u32x4 (&b)[2],
                                                  f32x16 c) {
  typedef int v8i32 __attribute__((ext_vector_type(8)));
  const v8i32 av = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3],
                    (int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
  const v8i32 bv = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                    (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
}

template <int N> using IC = std::integral_constant<int, N>;

// The epilogue's vector stores for a permuted B: within every wave's 32-row blocks, LDS rows
// I + 8g (I = 32j + 4h + e, g = 0..3) map to four consecutive logical columns.
template <RowPerm P, int MT_N>
constexpr bool epilogue_cols_ok() {
  if (P.block == 1) return true;
  for (int base = 0; base < MT_N; base += 32)
    for (int o = 0; o < 8; ++o)
      for (int g = 1; g < 4; ++g)
        if (P.fwd(base + o + 8 * g) != P.fwd(base + o) + g) return false;
  return true;
}
// The same for 64-column wave tiles whose LDS rows I + 16t (t = 0..3, I = 64w + o,
// o < 16) map to four consecutive logical columns (the fp8 transposed-operand permutation):
// a lane's values of blocks j = 0, 1 and groups g, g + 2 form one run.
template <RowPerm P, int MT_N, int WT_N>
constexpr bool epilogue_runs16_ok() {
  if (P.block == 1 || WT_N != 64) return false;
  for (int base = 0; base < MT_N; base += 64)
    for (int o = 0; o < 16; ++o)
      for (int t = 1; t < 4; ++t)
        if (P.fwd(base + o + 16 * t) != P.fwd(base + o) + t) return false;
  return true;
}

template <class T, bool A_KC, bool B_KC, bool U4B, int MT_M, int MT_N, int WM, int WN,
          int LROWS, int SCHED, int DTL, int MI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_tile_kernel(KArgs a) {
  using Cfg = TileCfg<T, A_KC, B_KC, U4B, MT_M, MT_N, WM, WN, LROWS, DTL, MI>;
  static_assert(MI == 32 || SCHED == 1, "16x16x32 blocks: ping-pong schedule");
  using OpA = typename Cfg::OpA;
  using OpB = typename Cfg::OpB;
  constexpr int BK = Cfg::BK, THREADS = Cfg::THREADS;
  constexpr int PA16 = Cfg::PA16, PB16 = Cfg::PB16;
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  constexpr int SA = Cfg::SA, SB = Cfg::SB;
  constexpr int SA1 = SA > 0 ? SA : 1, SB1 = SB > 0 ? SB : 1;  // array extents
  constexpr int EB = Cfg::EB;
  constexpr RowPerm PA = Cfg::PA, PB = Cfg::PB;
  constexpr int LDS_ALLOC = Cfg::lds_alloc(SCHED);
  __shared__ __attribute__((aligned(16))) u32x4 lds[LDS_ALLOC / 16];
  char* const ldsb = reinterpret_cast<char*>(lds);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile index: XCD-aware remap (consecutive workgroup ids go round-robin over the
  // 8 XCDs; give each XCD a contiguous range of tiles), then groups of 4 tile rows.
  const int tiles = a.tiles_m * a.tiles_n;
  int t = blockIdx.x;
  if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
  constexpr int GROUP_M = 4;
  const int group = GROUP_M * a.tiles_n;
  const int first_m = (t / group) * GROUP_M;
  const int gsz = min(a.tiles_m - first_m, GROUP_M);
  const int tile_m = first_m + (t % group) % gsz;
  const int tile_n = (t % group) / gsz;
  const int tile = tile_m * a.tiles_n + tile_n;
  const int m0 = tile_m * MT_M, n0 = tile_n * MT_N;

  const int z = blockIdx.z, sk = gridDim.z;
  const int kb = z * a.k_chunk;
  const int ke = min(a.K, kb + a.k_chunk);
  const int nt = ke > kb ? (ke - kb + BK - 1) / BK : 0;
  const int klen = ke - kb;

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.A, a.bytesA);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.B, a.bytesB);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.S, a.bytesS);

  Slot<OpA::VPB> sa[SA1];
  Slot<OpB::VPB> sb[SB1];
  typename Cfg::DA da;
  typename Cfg::DB db;
  typename Cfg::TA ta;
  typename Cfg::TB tb;
  if constexpr (Cfg::A_DTL) da.setup(lane, wave, m0, a.M, a.ldA, kb);
  if constexpr (Cfg::B_DTL) db.setup(lane, wave, n0, a.N, a.ldB, kb);
  if constexpr (Cfg::A_TR) ta.setup(lane, wave, m0, a.M, a.ldA, kb);
  if constexpr (Cfg::B_TR) tb.setup(lane, wave, n0, a.N, a.ldB, kb);
#pragma unroll
  for (int i = 0; i < SA; ++i) OpA::setup(sa[i], i * THREADS + tid, m0, a.M, a.ldA, kb, a.K);
#pragma unroll
  for (int i = 0; i < SB; ++i) OpB::setup(sb[i], i * THREADS + tid, n0, a.N, a.ldB, kb, a.K, a.b_tiled != 0);
  // Byte step of the offsets per K step.
  const uint32_t dA = A_KC ? BK * EB : (uint32_t)(BK * a.ldA) * EB;
  const uint32_t dB = U4B ? BK / 2u : (B_KC ? BK * EB : (uint32_t)(BK * a.ldB) * EB);

  // Register sets: with two, set (j % 2) holds the global data of K step j between its
  // loads (issued two steps ahead) and its LDS stores (one step ahead); with one, step j's
  // data is loaded and stored during step j-1.
  constexpr int NS = Cfg::NSETS;
  u32x4 ra[NS][SA1][OpA::VPB];
  u32x4 rb[NS][SB1][OpB::VPB];
  uint16_t rs[NS][SB1];

  // Direct-to-LDS loads of K step `step` into LDS buffer BUF.
  const u32x4 wA = rsrc_words(a.A, a.bytesA), wB = rsrc_words(a.B, a.bytesB);
  const uint32_t lds0 = lds_addr(ldsb);
  auto dtl = [&](int step, auto BUF_) {
    constexpr int BUF = decltype(BUF_)::value;
    const uint32_t sA = lds0 + BUF * Cfg::STAGE16 * 16;
    const int lim = klen - step * BK;
    if constexpr (Cfg::A_DTL) da.issue(wA, sA, wave, dA * (uint32_t)step, lim);
    if constexpr (Cfg::B_DTL) db.issue(wB, sA + Cfg::A16 * 16, wave, dB * (uint32_t)step, lim);
    if constexpr (Cfg::A_TR) ta.issue(wA, sA, wave, dA * (uint32_t)step, lim);
    if constexpr (Cfg::B_TR) tb.issue(wB, sA + Cfg::A16 * 16, wave, dB * (uint32_t)step, lim);
  };

  // Loads of K step `step` into set SET: vectors [J0, J1) of every block.
  auto load_part = [&](auto SET_, int step, auto J0_, auto J1_) {
    constexpr int SET = decltype(SET_)::value, J0 = decltype(J0_)::value, J1 = decltype(J1_)::value;
    const int lim = klen - step * BK;  // K indices left in the split from this step on
#pragma unroll
    for (int i = 0; i < SA; ++i) {
      const uint32_t d = dA * (uint32_t)step;
#pragma unroll
      for (int j = J0; j < J1 && j < OpA::VPB; ++j) {
        const bool ok = sa[i].kofs + (A_KC ? 0 : j) < lim;
        ra[SET][i][j] = ld128(rA, ok ? sa[i].off[j] + d : kOOB);
      }
    }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      // pre-tiled int4 codes: a 64-K step is half of a 4 KiB block's 64-byte rows
      const uint32_t d = (U4B && a.b_tiled) ? (uint32_t)(step >> 1) * 4096u + (uint32_t)(step & 1) * 32u
                                            : dB * (uint32_t)step;
#pragma unroll
      for (int j = J0; j < J1 && j < OpB::VPB; ++j) {
        const bool ok = sb[i].kofs + ((B_KC || U4B) ? 0 : j) < lim;
        rb[SET][i][j] = ld128(rB, ok ? sb[i].off[j] + d : kOOB);
        if constexpr (U4B) {
          const int gk = kb + step * BK + sb[i].kofs;
          rs[SET][i] = ld16b(rS, (ok && sb[i].row < a.N) ? ((uint32_t)(gk >> a.group_log2) * (uint32_t)a.N + sb[i].row) * 2u : kOOB);
        }
      }
    }
  };

  // LDS stores of set SET into buffer BUF, part P of 4 (vector P of a K-contiguous
  // block, transposed rows 2P and 2P+1, int4 chunk P).
  auto store_part = [&](auto SET_, auto BUF_, auto P_) {
    constexpr int SET = decltype(SET_)::value, BUF = decltype(BUF_)::value, P = decltype(P_)::value;
    char* sA = ldsb + BUF * Cfg::STAGE16 * 16;
    char* sB = sA + Cfg::A16 * 16;
#pragma unroll
    for (int i = 0; i < SA; ++i) {
      if constexpr (A_KC) {
        *reinterpret_cast<u32x4*>(sA + sa[i].wbase + P * (MT_M / 4) * OpA::PITCH_B) = ra[SET][i][P];
      } else if constexpr (Cfg::F8) {
        // elements 4P..4P+3 of the block's 16-byte vectors
        uint32_t o[4];
        transpose_bytes4(ra[SET][i][0][P], ra[SET][i][1][P], ra[SET][i][2][P], ra[SET][i][3][P], o);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint32_t*>(sA + sa[i].wbase + (4 * P + e) * OpA::ES * OpA::PITCH_B) = o[e];
      } else {
#pragma unroll
        for (int e = 2 * P; e < 2 * P + 2; ++e)
          *reinterpret_cast<u32x2*>(sA + sa[i].wbase + e * OpA::ES * OpA::PITCH_B) = transpose_row4(ra[SET][i], e);
      }
    }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if constexpr (U4B) {
        const _Float16 s = __builtin_bit_cast(_Float16, rs[SET][i]);
        const f16x2 s2 = {s, s};
        const _Float16 zb = (_Float16)(1024 + a.zero);
        const f16x2 bias = {zb, zb};
        *reinterpret_cast<u32x4*>(sB + sb[i].wbase + 16 * P) = dequant8(rb[SET][i][0][P], s2, bias);
      } else if constexpr (B_KC) {
        *reinterpret_cast<u32x4*>(sB + sb[i].wbase + P * (MT_N / 4) * OpB::PITCH_B) = rb[SET][i][P];
      } else if constexpr (Cfg::F8) {
        uint32_t o[4];
        transpose_bytes4(rb[SET][i][0][P], rb[SET][i][1][P], rb[SET][i][2][P], rb[SET][i][3][P], o);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint32_t*>(sB + sb[i].wbase + (4 * P + e) * OpB::ES * OpB::PITCH_B) = o[e];
      } else {
#pragma unroll
        for (int e = 2 * P; e < 2 * P + 2; ++e)
          *reinterpret_cast<u32x2*>(sB + sb[i].wbase + e * OpB::ES * OpB::PITCH_B) = transpose_row4(rb[SET][i], e);
      }
    }
  };

  // accumulators: one 32x32 (16 floats per lane) or 16x16 (4 floats per lane) block each
  using AccT = std::conditional_t<MI == 16, f32x4, f32x16>;
  constexpr int ACC_LEN = MI == 16 ? 4 : 16;
  AccT acc[TM * TN];
#pragma unroll
  for (int i = 0; i < TM * TN; ++i)
#pragma unroll
    for (int e = 0; e < ACC_LEN; ++e) acc[i][e] = 0.f;

  // Fragment reads (v_mfma_f32_32x32x16): lane reads LDS row (32-row block base +
  // lane%32), 16-byte chunk 2*kk + lane/32 of the step's K sub-step kk.
  // Per 16-K sub-step kk, in 16-byte units (stage-relative); block i adds 32 rows.
  const int r32 = lane & 31, kh = lane >> 5;
  int a_rd[4], b_rd[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int ca = Cfg::A_DTL ? ((2 * kk + kh) ^ dtl_swz(r32)) : 2 * kk + kh;
    const int cb = Cfg::B_DTL ? ((2 * kk + kh) ^ dtl_swz(r32)) : 2 * kk + kh;
    a_rd[kk] = (wm * Cfg::WT_M + r32) * PA16 + ca;
    b_rd[kk] = Cfg::A16 + (wn * Cfg::WT_N + r32) * PB16 + cb;
  }
  // 16x16x32 fragments: lane reads LDS row (16-row block base + lane%16), 16-byte chunk
  // 4h + lane/16 of the step's 32-K half h; block i adds 16 rows.
  const int r16 = lane & 15, kq = lane >> 4;
  int a_rd16[2], b_rd16[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // (16-aligned blocks: a lane's row bits below 4 are those of r16)
    const int csa = Cfg::CSWZ_A ? ((r16 >> 2) & 1) : 0, csb = Cfg::CSWZ_B ? ((r16 >> 2) & 1) : 0;
    const int ca = Cfg::A_DTL ? ((4 * h + kq) ^ dtl_swz(r16)) : ((4 * h + kq) ^ csa);
    const int cb = Cfg::B_DTL ? ((4 * h + kq) ^ dtl_swz(r16)) : ((4 * h + kq) ^ csb);
    a_rd16[h] = (wm * Cfg::WT_M + r16) * PA16 + ca;
    b_rd16[h] = Cfg::A16 + (wn * Cfg::WT_N + r16) * PB16 + cb;
  }
  // Transposed direct-to-LDS operands: byte offsets of the transposing reads, per block.
  int a_tr[TM], b_tr[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if constexpr (MI == 16 && Cfg::A_TR) a_tr[i] = Cfg::TA::frag_off16(lane, wm * Cfg::WT_M + 16 * i);
    else a_tr[i] = Cfg::TA::frag_off(lane, wm * Cfg::WT_M + 32 * i);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if constexpr (MI == 16 && Cfg::B_TR)
      b_tr[j] = Cfg::A16 * 16 + Cfg::TB::frag_off16(lane, wn * Cfg::WT_N + 16 * j);
    else
      b_tr[j] = Cfg::A16 * 16 + Cfg::TB::frag_off(lane, wn * Cfg::WT_N + 32 * j);
  }

  // Instruction counts of one sub-step, for the interleaving below.
  constexpr int N_MFMA = TM * TN;
  constexpr int N_READ = TM + TN;
  constexpr int TW = Cfg::F8 ? 4 : 2;   // LDS stores per part of a transposed block
  constexpr int N_WRITE = SA * (A_KC ? 1 : TW) + SB * (U4B ? 1 : (B_KC ? 1 : TW));
  constexpr int N_VMEM = SA + SB * (U4B ? 2 : 1);

  // K step s from LDS buffer CUR (= s % 2), four 16-K sub-steps kk. Sub-step kk also
  // issues the fragment reads of sub-step kk+1, vector kk of every block of step s+2
  // (into register set CUR, free since its data went to LDS last step) if LOAD, and part
  // kk of the LDS stores of step s+1 (set CUR^1 -> buffer CUR^1, free since it was read
  // last step) if STORE. The flags are compile-time so the loop body has no branches (a
  // branch would make the compiler wait for every outstanding load at the join), and
  // scheduling groups interleave the memory and permute work between the matrix-core
  // instructions so it runs while they execute.
  auto step = [&](int s, auto CUR_, auto LOAD_, auto STORE_) {
    constexpr int CUR = decltype(CUR_)::value;
    constexpr bool LOAD = decltype(LOAD_)::value, STORE = decltype(STORE_)::value;
    const u32x4* st = lds + CUR * Cfg::STAGE16;
    u32x4 fa[2][TM], fb[2][TN];
    auto read = [&](auto KK_) {
      constexpr int kk = decltype(KK_)::value;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (Cfg::A_TR)
          fa[kk & 1][i] = tr_fragment<Cfg::TA::R1>(reinterpret_cast<const char*>(st) + a_tr[i] +
                                                   Cfg::TA::KK_BYTES * kk);
        else
          fa[kk & 1][i] = st[a_rd[kk] + i * 32 * PA16];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (Cfg::B_TR)
          fb[kk & 1][j] = tr_fragment<Cfg::TB::R1>(reinterpret_cast<const char*>(st) + b_tr[j] +
                                                   Cfg::TB::KK_BYTES * kk);
        else
          fb[kk & 1][j] = st[b_rd[kk] + j * 32 * PB16];
      }
    };
    auto sub = [&](auto KK_) {
      constexpr int kk = decltype(KK_)::value;
      if constexpr (kk < 3) read(IC<kk + 1>{});
      if constexpr (NS == 2) {
        if constexpr (LOAD) load_part(CUR_, s + 2, IC<kk>{}, IC<kk + 1>{});
        if constexpr (STORE) store_part(IC<CUR ^ 1>{}, IC<CUR ^ 1>{}, KK_);
      } else {
        if constexpr (LOAD && kk == 0) load_part(IC<0>{}, s + 1, IC<0>{}, IC<4>{});
        if constexpr (STORE && kk >= 2) {
          store_part(IC<0>{}, IC<CUR ^ 1>{}, IC<2 * (kk - 2)>{});
          store_part(IC<0>{}, IC<CUR ^ 1>{}, IC<2 * (kk - 2) + 1>{});
        }
      }
      constexpr int n_vmem = NS == 2 ? N_VMEM : (kk == 0 ? 4 * N_VMEM : 0);
      constexpr int n_write = NS == 2 ? N_WRITE : (kk >= 2 ? 2 * N_WRITE : 0);
      if constexpr (MI == 32) {   // (the 16x16x32 kernels run the ping-pong schedule only)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i * TN + j] = mfma32x32x16<T>(fb[kk & 1][j], fa[kk & 1][i], acc[i * TN + j]);
      }
      // one matrix-core instruction, then a share of the other work, repeated
#pragma unroll
      for (int g = 0; g < N_MFMA; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
        if (kk < 3 && g < N_READ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        if (STORE && g < n_write) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        if (LOAD && g < n_vmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);                          // VALU
      }
    };
    static_assert(BK / 16 == 4, "four 16-K sub-steps per step");
    read(IC<0>{});
    if constexpr (Cfg::ANY_DTL) {
      // Step s+1 straight into the other LDS buffer (its last reads were in step s-1,
      // before the previous barrier), then the register loads of step s+2 (set CUR was
      // stored during step s-1): both have the whole step to land before the wait that
      // ends it.
      dtl(s + 1, IC<CUR ^ 1>{});
      load_part(CUR_, s + 2, IC<0>{}, IC<4>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    sub(IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
    oversync_point();
    sub(IC<1>{});
    __builtin_amdgcn_sched_barrier(0);
    oversync_point();
    sub(IC<2>{});
    __builtin_amdgcn_sched_barrier(0);
    oversync_point();
    sub(IC<3>{});
    oversync_point();
    if constexpr (Cfg::ANY_DTL) __builtin_amdgcn_s_waitcnt(0);  // every load of the step
    __syncthreads();
  };

  // fp8 K step s (128 K): two 64-K halves h, one v_mfma_f32_32x32x64 per 32x32 block and
  // half. A lane's 32-byte fragment of half h is its row's 16-byte chunks 4h + kh and
  // 4h + 2 + kh (the chunks the 16-bit sub-steps 2h and 2h + 1 read): A and B take the
  // same chunks, so both put the same K index in the same fragment byte and the products
  // pair up exactly whatever K order the instruction uses inside the fragment.
  // One register set per fragment (as many registers as the 16-bit double-buffered
  // sub-steps): half 0 walks the blocks in a snake, column 0 down then column 1 up, so
  // B fragment 0 and then the A fragments TM-1 .. 0 and B fragment 1 fall free one by one
  // and are reloaded with half 1's chunks right there; half 1 walks column 0 up, then
  // column 1 down, using them in the order they were reloaded (three or more multiplies
  // after each reload). Loads and stores of the next steps are spread over both halves.
  auto step8 = [&](int s, auto CUR_, auto LOAD_, auto STORE_) {
    constexpr int CUR = decltype(CUR_)::value;
    constexpr bool LOAD = decltype(LOAD_)::value, STORE = decltype(STORE_)::value;
    static_assert(NS == 2, "fp8 steps keep loads two steps ahead");
    static_assert(TN == 2, "the snake order is written for two B blocks per wave");
    const u32x4* st = lds + CUR * Cfg::STAGE16;
    u32x4 fa[TM][2], fb[TN][2];
    auto read_a = [&](int i, auto H_) {
      constexpr int H = decltype(H_)::value;
      fa[i][0] = st[a_rd[2 * H] + i * 32 * PA16];
      fa[i][1] = st[a_rd[2 * H + 1] + i * 32 * PA16];
    };
    auto read_b = [&](int j, auto H_) {
      constexpr int H = decltype(H_)::value;
      fb[j][0] = st[b_rd[2 * H] + j * 32 * PB16];
      fb[j][1] = st[b_rd[2 * H + 1] + j * 32 * PB16];
    };
    auto mma = [&](int i, int j) {
      if constexpr (MI == 32) acc[i * TN + j] = mfma32x32x64_f8(fb[j], fa[i], acc[i * TN + j]);
    };
    // Slot g of a half: one multiply, then that slot's share of the stores and loads.
    auto slots = [&](auto H_) {
      constexpr int H = decltype(H_)::value;
#pragma unroll
      for (int g = 0; g < N_MFMA; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                            // MFMA
        // half 0: reloads after the last use of B 0 (slot TM-1), of A TM-1..0 (slots
        // TM..2TM-1) and of B 1 (slot 2TM-1)
        if (H == 0 && g >= TM - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        if (H == 0 && g == N_MFMA - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int t = 0; t < (2 * N_WRITE) / N_MFMA + (g < (2 * N_WRITE) % N_MFMA ? 1 : 0); ++t)
          if (STORE) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);               // DS write
#pragma unroll
        for (int t = 0; t < (2 * N_VMEM) / N_MFMA + (g < (2 * N_VMEM) % N_MFMA ? 1 : 0); ++t)
          if (LOAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                            // VALU
      }
    };
    read_b(0, IC<0>{});
#pragma unroll
    for (int i = 0; i < TM; ++i) read_a(i, IC<0>{});
    read_b(1, IC<0>{});
    if constexpr (Cfg::ANY_DTL) {
      dtl(s + 1, IC<CUR ^ 1>{});
      load_part(CUR_, s + 2, IC<0>{}, IC<4>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    // half 0
    if constexpr (LOAD) load_part(CUR_, s + 2, IC<0>{}, IC<2>{});
    if constexpr (STORE) {
      store_part(IC<CUR ^ 1>{}, IC<CUR ^ 1>{}, IC<0>{});
      store_part(IC<CUR ^ 1>{}, IC<CUR ^ 1>{}, IC<1>{});
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) mma(i, 0);
    read_b(0, IC<1>{});
#pragma unroll
    for (int i = TM - 1; i >= 0; --i) {
      mma(i, 1);
      read_a(i, IC<1>{});
    }
    read_b(1, IC<1>{});
    slots(IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
    oversync_point();
    // half 1
    if constexpr (LOAD) load_part(CUR_, s + 2, IC<2>{}, IC<4>{});
    if constexpr (STORE) {
      store_part(IC<CUR ^ 1>{}, IC<CUR ^ 1>{}, IC<2>{});
      store_part(IC<CUR ^ 1>{}, IC<CUR ^ 1>{}, IC<3>{});
    }
#pragma unroll
    for (int i = TM - 1; i >= 0; --i) mma(i, 0);
#pragma unroll
    for (int i = 0; i < TM; ++i) mma(i, 1);
    slots(IC<1>{});
    if constexpr (Cfg::ANY_DTL) __builtin_amdgcn_s_waitcnt(0);  // every load of the step
    __syncthreads();
  };
  auto run_step = [&](int s, auto CUR_, auto LOAD_, auto STORE_) {
    if constexpr (Cfg::F8) step8(s, CUR_, LOAD_, STORE_);
    else step(s, CUR_, LOAD_, STORE_);
  };

  using TRUE = std::integral_constant<bool, true>;
  if constexpr (SCHED == 0) {
    // Every step loads two ahead and stores one ahead; loads past the split's end use
    // out-of-range offsets and return zeros, so the loop runs an even number of steps (a
    // padding step multiplies zeros and leaves the sums exact) and has no drain code.
    if constexpr (Cfg::ANY_DTL) {
      dtl(0, IC<0>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    load_part(IC<0>{}, 0, IC<0>{}, IC<4>{});
    if constexpr (NS == 2) load_part(IC<NS - 1>{}, 1, IC<0>{}, IC<4>{});
    store_part(IC<0>{}, IC<0>{}, IC<0>{});
    store_part(IC<0>{}, IC<0>{}, IC<1>{});
    store_part(IC<0>{}, IC<0>{}, IC<2>{});
    store_part(IC<0>{}, IC<0>{}, IC<3>{});
    if constexpr (Cfg::ANY_DTL) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    using LOADS = std::integral_constant<bool, !Cfg::ANY_DTL>;  // else issued at step start
    for (int s = 0; s < nt; s += 2) {
      run_step(s, IC<0>{}, LOADS{}, TRUE{});
      run_step(s + 1, IC<1>{}, LOADS{}, TRUE{});
    }
  } else if constexpr (SCHED == 2) {
    // One wave per SIMD (4 waves of 128x128), every operand straight into LDS, one barrier
    // per step, placed after sub-step 2. Per step s (LDS buffer CUR = s % 2):
    //   sub-step 0: 16 multiplies on fragment set 0; read sub-step 1's fragments (set 1)
    //   sub-step 1: 16 multiplies on set 1; read sub-step 2's fragments (set 0)
    //   sub-step 2: 16 multiplies on set 0; read sub-step 3's fragments (set 1)
    //   wait for this wave's direct loads (step s+1, issued a step ago) and its reads; barrier
    //   sub-step 3: 16 multiplies on set 1; read step s+1's sub-step 0 fragments from the
    //               other buffer (set 0); issue step s+2's direct loads into buffer CUR
    // After the barrier of step s every wave has finished reading buffer CUR (its last
    // reads completed before the barrier) and every wave's loads of step s+1 have landed,
    // so sub-step 3 can both read step s+1 and refill buffer CUR with step s+2. The
    // matrix cores never wait for a read issued after a barrier: the 16 multiplies of
    // sub-step 3 use fragments read before it.
    static_assert(SA == 0 && SB == 0 && !Cfg::F8 && NS == 2, "every operand direct-to-LDS, 16-bit");
    constexpr int NIA = Cfg::A_DTL ? Cfg::DA::NI : (Cfg::A_TR ? Cfg::TA::NI : 0);
    constexpr int NIB = Cfg::B_DTL ? Cfg::DB::NI : (Cfg::B_TR ? Cfg::TB::NI : 0);
    constexpr int NLD = NIA + NIB;   // direct loads per wave and step
    constexpr int NMF = TM * TN;     // multiplies per sub-step
    u32x4 fa[2][TM], fb[2][TN];
    auto read_frag = [&](int buf, int kk, int q, int f) {
      // fragment f of sub-step kk: A blocks 0..TM-1, then B blocks 0..TN-1
      const u32x4* st = lds + buf * Cfg::STAGE16;
      const char* sbytes = reinterpret_cast<const char*>(st);
      if (f < TM) {
        const int i = f;
        if constexpr (Cfg::A_TR)
          fa[q][i] = tr_fragment<Cfg::TA::R1>(sbytes + a_tr[i] + Cfg::TA::KK_BYTES * kk);
        else
          fa[q][i] = st[a_rd[kk] + i * 32 * PA16];
      } else {
        const int j = f - TM;
        if constexpr (Cfg::B_TR)
          fb[q][j] = tr_fragment<Cfg::TB::R1>(sbytes + b_tr[j] + Cfg::TB::KK_BYTES * kk);
        else
          fb[q][j] = st[b_rd[kk] + j * 32 * PB16];
      }
    };
    auto dtl_one = [&](int step, int buf, int g) {
      const uint32_t sA = lds0 + buf * Cfg::STAGE16 * 16;
      const int lim = klen - step * BK;
      if (g < NIA) {
        if constexpr (Cfg::A_DTL) da.issue_one(wA, sA, wave, dA * (uint32_t)step, lim, g);
        if constexpr (Cfg::A_TR) ta.issue_one(wA, sA, wave, dA * (uint32_t)step, lim, g);
      } else {
        if constexpr (Cfg::B_DTL) db.issue_one(wB, sA + Cfg::A16 * 16, wave, dB * (uint32_t)step, lim, g - NIA);
        if constexpr (Cfg::B_TR) tb.issue_one(wB, sA + Cfg::A16 * 16, wave, dB * (uint32_t)step, lim, g - NIA);
      }
    };
    // Sub-step kk of a step in buffer CUR: multiply set Q, and after the multiply g, read
    // fragment g of the next sub-step (from buffer RBUF, sub-step RKK, into set Q ^ 1) and,
    // in sub-step 3, issue the direct loads of step s + 2 into buffer CUR (load l after
    // multiply l * NMF / NLD).
    auto substep = [&](int s, auto CUR_, auto KK_) {
      constexpr int CUR = decltype(CUR_)::value, kk = decltype(KK_)::value;
      constexpr int Q = kk & 1;
      constexpr int RBUF = kk < 3 ? CUR : CUR ^ 1, RKK = (kk + 1) & 3;
#pragma unroll
      for (int g = 0; g < TM * TN; ++g) {
        const int i = g / TN, j = g % TN;
        acc[i * TN + j] = mfma32x32x16<T>(fb[Q][j], fa[Q][i], acc[i * TN + j]);
        if (g < TM + TN) read_frag(RBUF, RKK, Q ^ 1, g);
        if constexpr (kk == 3) {
          // the step's direct loads spread evenly over the sub-step's multiplies
#pragma unroll
          for (int l = g * NLD / NMF; l < (g + 1) * NLD / NMF; ++l) dtl_one(s + 2, CUR, l);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto step_w4 = [&](int s, auto CUR_) {
      substep(s, CUR_, IC<0>{});
      substep(s, CUR_, IC<1>{});
      substep(s, CUR_, IC<2>{});
      oversync_point();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of step s+1 and its reads of step s
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      substep(s, CUR_, IC<3>{});
      oversync_point();
    };
    dtl(0, IC<0>{});
    dtl(1, IC<1>{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((NLD & 15) | (7 << 4) | (15 << 8) | (((NLD >> 4) & 3) << 14));  // step 0 landed
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < TM + TN; ++f) read_frag(0, 0, 0, f);
    for (int s = 0; s < nt; s += 2) {
      // two steps per iteration so the buffer indices are compile-time; an odd step count
      // ends with a step of zeros (its loads lie past the split)
      step_w4(s, IC<0>{});
      step_w4(s + 1, IC<1>{});
    }
    // the last direct loads (zeros past the split) still write LDS, which the epilogue
    // reuses: every wave waits for its own, then one more barrier for all
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  } else {
    // Ping-pong schedule. The waves form two groups (wave rows wm = 0 and 1, one wave of
    // each on every SIMD) that run the same program one phase apart, so in every phase
    // one wave per SIMD issues matrix-core instructions on fragments already in
    // registers while the other reads its next fragments from LDS and, once per step,
    // transposes and stores the next step's tile and issues the global loads of the one
    // after. Per step and wave: C(first half of K) | M(read second half; store step s+1;
    // load step s+2) | C(second half) | M(read first half of step s+1), with a barrier
    // after every phase. Group 1 starts one barrier late and group 0 ends with one extra
    // barrier, so both execute the same number of barriers.
    // K-contiguous operands go straight into LDS instead (direct-to-LDS loads, no
    // registers and no LDS stores of the threads), and so do transposed operands in the
    // variant that transposes them with the LDS reads. A wave issues its share of step t's
    // direct loads in the memory phase that only reads, between the last compute phase of
    // step t-2 and the first of step t-1: two barriers after the last read of that buffer
    // by either group.
    // It waits for them at the end of its next storing memory phase, which comes before
    // the barrier ahead of the first read of step t by either group.
    static_assert(WM == 2 && NS == 2, "ping-pong layout: two wave rows, one block per operand");
    const int grp = wm;
    u32x4 fa[2][TM], fb[2][TN];
    auto readh = [&](int buf, auto H_) {
      constexpr int H = decltype(H_)::value;
      const u32x4* st = lds + buf * Cfg::STAGE16;
      const char* sbytes = reinterpret_cast<const char*>(st);
      if constexpr (MI == 16) {   // one 16x16x32 fragment per block covers the half
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if constexpr (Cfg::A_TR)
            fa[0][i] = tr_fragment<Cfg::TA::R1>(sbytes + a_tr[i] + Cfg::TA::KK16_BYTES * H);
          else
            fa[0][i] = st[a_rd16[H] + i * 16 * PA16];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (Cfg::B_TR)
            fb[0][j] = tr_fragment<Cfg::TB::R1>(sbytes + b_tr[j] + Cfg::TB::KK16_BYTES * H);
          else
            fb[0][j] = st[b_rd16[H] + j * 16 * PB16];
        }
        return;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if constexpr (Cfg::A_TR)
            fa[q][i] = tr_fragment<Cfg::TA::R1>(sbytes + a_tr[i] + Cfg::TA::KK_BYTES * (2 * H + q));
          else
            fa[q][i] = st[a_rd[2 * H + q] + i * 32 * PA16];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (Cfg::B_TR)
            fb[q][j] = tr_fragment<Cfg::TB::R1>(sbytes + b_tr[j] + Cfg::TB::KK_BYTES * (2 * H + q));
          else
            fb[q][j] = st[b_rd[2 * H + q] + j * 32 * PB16];
        }
      }
    };
    auto compute = [&]() {
      if constexpr (MI == 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i * TN + j] = mfma16x16x32<T>(fb[0][j], fa[0][i], acc[i * TN + j]);
      } else if constexpr (Cfg::F8) {
        // one 32x32x64 multiply per block and half: its 32-byte fragment is the half's two
        // 16-byte chunks, read as for the two 16-bit sub-steps (same chunks on A and B, so
        // the products pair up as in the fp8 pipeline step)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const u32x4 a2[2] = {fa[0][i], fa[1][i]};
            const u32x4 b2[2] = {fb[0][j], fb[1][j]};
            acc[i * TN + j] = mfma32x32x64_f8(b2, a2, acc[i * TN + j]);
          }
      } else {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i * TN + j] = mfma32x32x16<T>(fb[q][j], fa[q][i], acc[i * TN + j]);
      }
    };
    // Barrier between phases, fenced so the scheduler cannot move matrix-core or memory
    // instructions from one phase into another (MFMAs have no memory effects and would
    // otherwise drift across a plain barrier).
    auto phase_barrier = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kOverSync) __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto store_all = [&](int buf) {
      if (buf == 0) {
        store_part(IC<0>{}, IC<0>{}, IC<0>{});
        store_part(IC<0>{}, IC<0>{}, IC<1>{});
        store_part(IC<0>{}, IC<0>{}, IC<2>{});
        store_part(IC<0>{}, IC<0>{}, IC<3>{});
      } else {
        store_part(IC<0>{}, IC<1>{}, IC<0>{});
        store_part(IC<0>{}, IC<1>{}, IC<1>{});
        store_part(IC<0>{}, IC<1>{}, IC<2>{});
        store_part(IC<0>{}, IC<1>{}, IC<3>{});
      }
    };
    // register loads per load_part (int4 B: a scale load per code vector too) and this
    // wave's direct-to-LDS loads per step
    constexpr int NREG = SA * OpA::VPB + SB * OpB::VPB * (U4B ? 2 : 1);
    constexpr int NDTL = (Cfg::A_DTL ? Cfg::DA::NI : 0) + (Cfg::B_DTL ? Cfg::DB::NI : 0) +
                         (Cfg::A_TR ? Cfg::TA::NI : 0) + (Cfg::B_TR ? Cfg::TB::NI : 0);
    static_assert(NREG + NDTL < 64, "vmcnt field");
    // s_waitcnt vmcnt(N), no wait on the other counters. The count is by issue order: every
    // load before the wait except the N most recent has landed. Fenced so that the loads
    // the count assumes stay before the wait.
    auto wait_vm = [](auto N_) {
      constexpr int n = decltype(N_)::value;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14));
      __builtin_amdgcn_sched_barrier(0);
    };
    auto dtl_fenced = [&](int step, auto BUF_) {
      __builtin_amdgcn_sched_barrier(0);
      dtl(step, BUF_);
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (Cfg::ANY_DTL) dtl_fenced(0, IC<0>{});
    load_part(IC<0>{}, 0, IC<0>{}, IC<4>{});
    store_all(0);
    load_part(IC<0>{}, 1, IC<0>{}, IC<4>{});
    if constexpr (Cfg::ANY_DTL) {
      dtl_fenced(1, IC<1>{});        // buffer 1 has not been used yet
      wait_vm(IC<NREG + NDTL>{});    // step 0 in LDS; step 1's loads may still fly
    }
    phase_barrier();
    if (grp == 1) phase_barrier();
    readh(0, IC<0>{});
    phase_barrier();
    for (int s = 0; s < nt; s += 2) {
      // two steps per iteration so the buffer indices are compile-time
      compute();
      phase_barrier();
      readh(0, IC<1>{});
      store_all(1);
      load_part(IC<0>{}, s + 2, IC<0>{}, IC<4>{});
      if constexpr (Cfg::ANY_DTL) wait_vm(IC<NREG>{});   // step s+1's direct loads
      phase_barrier();
      compute();
      phase_barrier();
      readh(1, IC<0>{});
      if constexpr (Cfg::ANY_DTL) dtl_fenced(s + 2, IC<0>{});
      phase_barrier();
      compute();
      phase_barrier();
      readh(1, IC<1>{});
      store_all(0);
      load_part(IC<0>{}, s + 3, IC<0>{}, IC<4>{});
      if constexpr (Cfg::ANY_DTL) wait_vm(IC<NREG>{});   // step s+2's direct loads
      phase_barrier();
      compute();
      phase_barrier();
      readh(0, IC<0>{});
      if constexpr (Cfg::ANY_DTL) dtl_fenced(s + 3, IC<1>{});
      phase_barrier();
    }
    if (grp == 0) phase_barrier();
    if constexpr (Cfg::ANY_DTL) {
      // the last direct loads (zeros past the split) still write LDS, which the epilogue
      // reuses: every wave waits for its own, then one more barrier for all
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // (schedule 2 is planned without split-K: its 256 accumulators leave no registers for
  // the fix-up's element-wise sums)
  if constexpr (SCHED != 2) {
    if (sk > 1) {
      if (!splitk_fixup<AccT, TM * TN, THREADS>(acc, a, tile, z, sk, tiles)) return;
    }
  }

  // ---- epilogue: block (i, j), lane l holds logical row fwd_A(LDS row 32i + l%32) and,
  // for g = 0..3, the four logical columns fwd_B(LDS rows 32j + 8g + 4(l/32) + 0..3)
  // (16x16x32 blocks: LDS row 16i + l%16 and the columns fwd_B(LDS rows 16j + 4(l/16) +
  // 0..3)). The C tile is staged in LDS by A's LDS row (consecutive lanes on
  // consecutive rows, so the stores spread over the banks) and each staged row goes to
  // global row fwd_A(row) in 16-byte pieces, whole rows per pass (measured 2-5% faster
  // than storing four-element vectors straight from the accumulators).
  constexpr bool COLS4 = epilogue_cols_ok<PB, MT_N>();
  constexpr bool RUNS16 = !COLS4 && epilogue_runs16_ok<PB, MT_N, Cfg::WT_N>();
  // 16x16x32 blocks, B transposed in registers (64-row, stride-8 rows), one permutation block
  // per wave: lane pairs (l, l + 32) exchange values to store whole column runs (below)
  constexpr bool PAIR16 = MI == 16 && PB.block == 64 && PB.stride == 8 && Cfg::WT_N == 64 && TN == 4;
  auto epilogue = [&](auto dt_tag) {
    constexpr int DT = decltype(dt_tag)::value;
    using O = typename OutT<DT>::type;
    constexpr int OB = OutT<DT>::bytes;
    constexpr int ROW_BYTES = MT_N * OB;
    constexpr int CP = ROW_BYTES + 16;                    // LDS pitch of the C tile
    constexpr int RPP0 = LDS_ALLOC / CP;
    constexpr int RPP = RPP0 >= MT_M ? MT_M : (RPP0 / 32) * 32;  // rows per pass
    constexpr int NPASS = (MT_M + RPP - 1) / RPP;
    constexpr int CPR = ROW_BYTES / 16;                   // 16-byte chunks per row
    char* cl = reinterpret_cast<char*>(lds);
    O* Cg = reinterpret_cast<O*>(a.C);
#pragma unroll 1
    for (int p = 0; p < NPASS; ++p) {
      const int lo = p * RPP;
      if constexpr (MI == 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int m = wm * Cfg::WT_M + i * 16 + r16;   // LDS row of A
          if (m < lo || m >= lo + RPP) continue;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int nb = wn * Cfg::WT_N + j * 16 + 4 * kq;
            const auto& v = acc[i * TN + j];
            if constexpr (PB.block == 1) {
              O* dst = reinterpret_cast<O*>(cl + (m - lo) * CP + nb * OB);
              typedef O o4 __attribute__((ext_vector_type(4)));
              o4 w = {cvt_out<DT>(v[0]), cvt_out<DT>(v[1]), cvt_out<DT>(v[2]), cvt_out<DT>(v[3])};
              *reinterpret_cast<o4*>(dst) = w;
            } else if constexpr (!PAIR16) {
              // B transposed in registers: its permuted LDS rows nb + e hold logical
              // columns fwd_B(nb + e), eight apart; one element each
#pragma unroll
              for (int e = 0; e < 4; ++e)
                *reinterpret_cast<O*>(cl + (m - lo) * CP + PB.fwd(nb + e) * OB) = cvt_out<DT>(v[e]);
            }
          }
          if constexpr (PAIR16) {
            // B transposed in registers, 64-row stride-8 permutation, one 64-row block per
            // wave: lane l (l < 32) holds logical columns 32(kq%2) + 8e + 2j and lane l + 32 the
            // columns one higher (e = 0..3, block j = 0..3). Two lane swaps per block give lane
            // l the 16 consecutive columns of e = 0, 1 and lane l + 32 those of e = 2, 3.
            float c16[16];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              // (copies to scalars first: a bit cast of a vector element reads element 0)
              const float v0 = acc[i * TN + j][0], v1 = acc[i * TN + j][1];
              const float v2 = acc[i * TN + j][2], v3 = acc[i * TN + j][3];
              const auto s0 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v0),
                                                               __builtin_bit_cast(unsigned, v2), false, false);
              const auto s1 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v1),
                                                               __builtin_bit_cast(unsigned, v3), false, false);
              const unsigned s00 = s0[0], s01 = s0[1], s10 = s1[0], s11 = s1[1];
              c16[2 * j] = __builtin_bit_cast(float, s00);
              c16[2 * j + 1] = __builtin_bit_cast(float, s01);
              c16[8 + 2 * j] = __builtin_bit_cast(float, s10);
              c16[8 + 2 * j + 1] = __builtin_bit_cast(float, s11);
            }
            const int col0 = wn * 64 + 32 * (kq % 2) + 16 * (kq / 2);
            typedef O o4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              o4 w = {cvt_out<DT>(c16[4 * q]), cvt_out<DT>(c16[4 * q + 1]), cvt_out<DT>(c16[4 * q + 2]),
                      cvt_out<DT>(c16[4 * q + 3])};
              *reinterpret_cast<o4*>(cl + (m - lo) * CP + (col0 + 4 * q) * OB) = w;
            }
          }
        }
      } else
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = wm * Cfg::WT_M + i * 32 + r32;   // LDS row of A
        if (m < lo || m >= lo + RPP) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int nb = wn * Cfg::WT_N + j * 32 + 8 * g + 4 * kh;
            const auto& v = acc[i * TN + j];   // (a 32x32 block: 16 floats)
            if constexpr (PB.block == 1) {
              O* dst = reinterpret_cast<O*>(cl + (m - lo) * CP + nb * OB);
              typedef O o4 __attribute__((ext_vector_type(4)));
              o4 w = {cvt_out<DT>(v[4 * g]), cvt_out<DT>(v[4 * g + 1]), cvt_out<DT>(v[4 * g + 2]),
                      cvt_out<DT>(v[4 * g + 3])};
              *reinterpret_cast<o4*>(dst) = w;
            } else if constexpr (COLS4) {
              if (g == 0) {
                // B's rows are permuted: LDS rows nb + e + 8g (g = 0..3) hold the four
                // consecutive logical columns fwd_B(nb + e) + g: one vector store per e.
                typedef O o4 __attribute__((ext_vector_type(4)));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  O* dst = reinterpret_cast<O*>(cl + (m - lo) * CP + PB.fwd(nb + e) * OB);
                  o4 w = {cvt_out<DT>(v[e]), cvt_out<DT>(v[4 + e]), cvt_out<DT>(v[8 + e]),
                          cvt_out<DT>(v[12 + e])};
                  *reinterpret_cast<o4*>(dst) = w;
                }
              }
            } else if constexpr (RUNS16) {
              if (j == 0 && g < 2) {
                // LDS rows nb + e + 16t, t = 2j' + g' (block j', group g + 2g'), hold the
                // logical columns fwd_B(nb + e) + t: one vector store per e.
                const auto& v1 = acc[i * TN + 1];
                typedef O o4 __attribute__((ext_vector_type(4)));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  O* dst = reinterpret_cast<O*>(cl + (m - lo) * CP + PB.fwd(nb + e) * OB);
                  o4 w = {cvt_out<DT>(v[4 * g + e]), cvt_out<DT>(v[4 * g + 8 + e]),
                          cvt_out<DT>(v1[4 * g + e]), cvt_out<DT>(v1[4 * g + 8 + e])};
                  *reinterpret_cast<o4*>(dst) = w;
                }
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                *reinterpret_cast<O*>(cl + (m - lo) * CP + PB.fwd(nb + e) * OB) = cvt_out<DT>(v[4 * g + e]);
            }
          }
        }
      }
      __syncthreads();
      const int rows = min(RPP, MT_M - lo);  // the last pass may be short
      for (int c = tid; c < rows * CPR; c += THREADS) {
        const int row = c / CPR, cc = c % CPR;
        const int gm = m0 + PA.fwd(lo + row);
        const int gn = n0 + cc * (16 / OB);
        if (gm >= a.M || gn >= a.N) continue;
        const char* src = cl + row * CP + cc * 16;
        if (a.c_vec && gn + 16 / OB <= a.N) {
          // non-temporal: C is not read again here (measured 0.5-0.7% faster at 4096^3)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src),
                                      reinterpret_cast<u32x4*>(Cg + (size_t)gm * a.N + gn));
        } else {
#pragma unroll
          for (int q = 0; q < 16 / OB; ++q)
            if (gn + q < a.N) Cg[(size_t)gm * a.N + gn + q] = reinterpret_cast<const O*>(src)[q];
        }
      }
      __syncthreads();
    }
  };
  // Schedule 2 (one wave of 128x128 per SIMD) stores C straight from the accumulators (its
  // 128x128 accumulators leave no registers for a second pass of the staged epilogue): lane
  // l of block (i, j) holds row 32i + l%32 and, for g = 0..3, the four consecutive columns
  // 32j + 8g + 4(l/32) + 0..3, so each store is one 4-element vector; the lanes of a store
  // cover 16 contiguous bytes of 32 rows (fp16), and the 16 stores of a block fill whole
  // 128-byte lines of those rows. No LDS round trip, and no accumulator needs to wait for a
  // second pass (the two-pass LDS epilogue of an fp32 tile would not fit the registers).
  auto epilogue_direct = [&](auto dt_tag) {
    constexpr int DT = decltype(dt_tag)::value;
    using O = typename OutT<DT>::type;
    typedef O o4 __attribute__((ext_vector_type(4)));
    O* Cg = reinterpret_cast<O*>(a.C);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int gm = m0 + wm * Cfg::WT_M + i * 32 + r32;
      if (gm >= a.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int gn = n0 + wn * Cfg::WT_N + j * 32 + 8 * g + 4 * kh;
          const auto& v = acc[i * TN + j];
          O* dst = Cg + (size_t)gm * a.N + gn;
          if (a.c_vec && gn + 4 <= a.N) {
            o4 w = {cvt_out<DT>(v[4 * g]), cvt_out<DT>(v[4 * g + 1]), cvt_out<DT>(v[4 * g + 2]),
                    cvt_out<DT>(v[4 * g + 3])};
            *reinterpret_cast<o4*>(dst) = w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gn + e < a.N) dst[e] = cvt_out<DT>(v[4 * g + e]);
          }
        }
      }
    }
  };
  if constexpr (SCHED == 2) {
    if (a.dtype_c == DT_F16) epilogue_direct(std::integral_constant<int, DT_F16>{});
    else if (a.dtype_c == DT_BF16) epilogue_direct(std::integral_constant<int, DT_BF16>{});
    else epilogue_direct(std::integral_constant<int, DT_F32>{});
  } else {
    // The C tile reuses the operand LDS: every wave is past the loop's last barrier.
    if (a.dtype_c == DT_F16) epilogue(std::integral_constant<int, DT_F16>{});
    else if (a.dtype_c == DT_BF16) epilogue(std::integral_constant<int, DT_BF16>{});
    else epilogue(std::integral_constant<int, DT_F32>{});
  }
}

// ================================================================= skinny kernel

// M <= 16, A row-major (K-contiguous), B column-major (K-contiguous) or int4 codes packed
// along K. Workgroup: W waves over one 16 x (16*NB) output tile. A wave iteration covers
// KI K indices: lane (r = lane%16, c = lane/16) loads, for B row n0+16*nb+r and A row r,
// the K range [k + c*KI/4, k + (c+1)*KI/4); matrix-core step h uses the lane's h-th group
// of eight K indices, identically for A and B, so the pairing of K indices is exact.
// Iterations are dealt to the waves in turn (iteration i to wave i % W), so at any time the
// workgroup reads one contiguous K window of every column.
// Main loop: two register sets of U iterations each. While one set is multiplied, the
// other set's loads are in flight, and each set is reloaded as soon as it has been used.
// The loop body has no branches: an iteration past the split's end loads with
// out-of-range offsets, which return zeros, and multiplies zeros. So the compiler can wait
// for exactly the loads each multiply needs (it counts outstanding loads in issue order)
// instead of for every outstanding load.
template <class T, bool U4B, int NB, int W, int U>
__global__ __launch_bounds__(W * 64) void gemm_skinny_kernel(KArgs a) {
  constexpr int THREADS = W * 64;
  constexpr int KI = U4B ? 128 : 64;   // K per wave iteration
  constexpr int H = KI / 32;           // matrix-core steps per iteration and n-block
  constexpr int KL = KI / 4;           // K indices per lane per iteration
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int tile = blockIdx.x;
  const int n0 = tile * 16 * NB;
  const int z = blockIdx.y, sk = gridDim.y;
  const int kb = z * a.k_chunk;
  const int ke = min(a.K, kb + a.k_chunk);
  const int n_it = ke > kb ? (ke - kb + KI - 1) / KI : 0;

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.A, a.bytesA);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.B, a.bytesB);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.S, a.bytesS);

  constexpr int BV = U4B ? 1 : H;      // 16-byte B vectors per lane per n-block
  u32x4 bufA[2][U][H];
  u32x4 bufB[2][U][NB][BV];
  uint16_t bufS[2][U][NB];

  // int4: every load of an iteration lies inside the split (split chunks are multiples of
  // 128 and K % 128 == 0) and rows past M or N start past the end of their buffer, where
  // buffer loads return zeros; so the offsets are per-lane constants plus a wave-uniform
  // per-iteration term (scalar offset), with no per-load bounds arithmetic. An iteration
  // past the split's end takes the scalar offset kOOB: every per-lane offset is below 2^31,
  // so the sum stays below 2^32 and lies past every buffer's end.
  uint32_t offA0 = 0, offB0[NB], offS0[NB];
  if constexpr (U4B) {
    // activations, coalesced: load h of an iteration takes rows 4h + lane/16, the 16-byte
    // chunk lane%16 of each row's 256 bytes (whole 128-byte lines, 1 KiB per load); the
    // fragments are then formed through the wave's LDS slot (transpose_a below)
    offA0 = (uint32_t)((lane >> 4) * a.ldA + kb + 8 * (lane & 15)) * 2u;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = n0 + 16 * nb + r;
      // column-major packing: byte n*(K/2) + k/2; pre-tiled: 4 KiB blocks of 64 columns x
      // 128 K (one iteration), 64 bytes per column
      offB0[nb] = a.b_tiled ? ((uint32_t)((n / 64) * (a.K / 128) + kb / 128) * 64u + (uint32_t)(n % 64)) * 64u + 16u * c
                            : (uint32_t)n * (uint32_t)(a.K / 2) + (uint32_t)((kb + c * KL) / 2);
      // scale row (kb + it * KI + c * KL) / group: kb + it * KI is a multiple of 128, so the
      // lane part c * KL and the iteration part separate (exact for every group >= 32)
      offS0[nb] = ((uint32_t)((c * KL) >> a.group_log2) * (uint32_t)a.N + (uint32_t)n) * 2u;
    }
  }
  const uint32_t b_iter = a.b_tiled ? 4096u : (uint32_t)(KI / 2);   // B bytes per iteration
  // Loads of iteration `it` of this split into slot u of register set SET.
  auto load = [&](auto SET_, int u, int it) {
    constexpr int SET = decltype(SET_)::value;
    const bool live = it < n_it;
    if constexpr (U4B) {
      const uint32_t sa = live ? (uint32_t)it * KI * 2u : kOOB;
      const uint32_t sb = live ? (uint32_t)it * b_iter : kOOB;
      const uint32_t ss = live ? (uint32_t)((kb + it * KI) >> a.group_log2) * (uint32_t)a.N * 2u : kOOB;
#pragma unroll
      for (int h = 0; h < H; ++h)
        bufA[SET][u][h] = __builtin_amdgcn_raw_buffer_load_b128(rA, offA0 + (uint32_t)(4 * h * a.ldA) * 2u, sa, 0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        bufB[SET][u][nb][0] = __builtin_amdgcn_raw_buffer_load_b128(rB, offB0[nb], sb, 0);
        bufS[SET][u][nb] = __builtin_amdgcn_raw_buffer_load_b16(rS, offS0[nb], ss, 0);
      }
      return;
    }
    const int k = kb + it * KI + c * KL;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const bool ok = live && r < a.M && k + 8 * h < ke;
      bufA[SET][u][h] = ld128(rA, ok ? (uint32_t)(r * a.ldA + k + 8 * h) * 2u : kOOB);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = n0 + 16 * nb + r;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const bool ok = live && n < a.N && k + 8 * h < ke;
        bufB[SET][u][nb][h] = ld128(rB, ok ? (uint32_t)(n * a.ldB + k + 8 * h) * 2u : kOOB);
      }
    }
  };

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const _Float16 zb = (_Float16)(-1024 - a.zero), zb16 = (_Float16)(-64 - a.zero);
  const f16x2 bias = {zb, zb}, bias16 = {zb16, zb16};
  // int4: the wave's LDS slot turns one iteration's coalesced activation loads (load h: rows
  // 4h + c', chunk r') into matrix-core fragments (fragment h: row r, chunk 4c + h, i.e. K
  // indices 32c + 8h .. +7, the K indices of the codes in dword h of the lane's 16 bytes).
  // The row pitch of 272 bytes puts the 16 rows a fragment read touches on 16 distinct
  // 16-byte bank groups. Only the wave itself uses its slot, and one wave's LDS accesses
  // complete in order, so no barrier is needed.
  constexpr int APITCH = 272;
  __shared__ __attribute__((aligned(16))) char aslot[U4B ? W : 1][U4B ? 16 * APITCH : 16];
  auto transpose_a = [&](const u32x4 (&v)[H], int h) {
    char* slot = aslot[U4B ? wave : 0];
    if (h == 0) {
#pragma unroll
      for (int g = 0; g < H; ++g)
        *reinterpret_cast<u32x4*>(slot + (4 * g + (lane >> 4)) * APITCH + 16 * (lane & 15)) = v[g];
    }
    return *reinterpret_cast<const u32x4*>(slot + r * APITCH + (4 * c + h) * 16);
  };
  auto compute = [&](auto SET_, int u) {
    constexpr int SET = decltype(SET_)::value;
    if constexpr (U4B) {
      // the activation fragments take the weights' K order (pairs k, k+4), once per
      // iteration for all NB blocks
      u32x4 ap[H];
#pragma unroll
      for (int h = 0; h < H; ++h) ap[h] = pair_k_and_k4(transpose_a(bufA[SET][u], h));
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const _Float16 s = __builtin_bit_cast(_Float16, bufS[SET][u][nb]);
          const f16x2 s2 = {s, s};
          acc[nb] = mfma16x16x32<T>(dequant8_pairs(bufB[SET][u][nb][0][h], s2, bias, bias16), ap[h], acc[nb]);
        }
    } else {
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb] = mfma16x16x32<T>(bufB[SET][u][nb][h], bufA[SET][u][h], acc[nb]);
    }
  };

  // iteration of slot u in round q (rounds of W*U iterations; round q uses set q % 2)
  auto iter = [&](int q, int u) { return q * (W * U) + u * W + wave; };
  const int rounds = (n_it + W * U - 1) / (W * U);
#pragma unroll
  for (int u = 0; u < U; ++u) load(IC<0>{}, u, iter(0, u));
#pragma unroll
  for (int u = 0; u < U; ++u) load(IC<1>{}, u, iter(1, u));
  for (int q = 0; q < rounds; q += 2) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      compute(IC<0>{}, u);
      load(IC<0>{}, u, iter(q + 2, u));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      compute(IC<1>{}, u);
      load(IC<1>{}, u, iter(q + 3, u));
    }
  }

  // ---- cross-wave reduction through LDS: wave w's partial tile -> red[w]; then each
  // thread sums, in wave order, the positions p = tid, tid + THREADS, ... below P
  constexpr int P = NB * 64;                     // f32x4 positions per tile
  constexpr int NV = (P + THREADS - 1) / THREADS;
  static_assert(P <= THREADS || P % THREADS == 0, "whole vectors of positions per thread");
  __shared__ f32x4 red[W][P];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) red[wave][nb * 64 + lane] = acc[nb];
  __syncthreads();
  f32x4 sum[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int p = v * THREADS + tid;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p < P) {
      s = red[0][p];
#pragma unroll
      for (int w = 1; w < W; ++w) s += red[w][p];
    }
    sum[v] = s;
  }

  if (sk > 1) {
    if (!splitk_fixup<f32x4, NV, THREADS, (P < THREADS ? P : THREADS)>(sum, a, tile, z, sk, gridDim.x)) return;
  }

  // ---- store: position p = nb*64 + l holds row l%16, columns n0 + 16nb + 4(l/16) + 0..3
  auto store = [&](auto dt_tag) {
    constexpr int DT = decltype(dt_tag)::value;
    using O = typename OutT<DT>::type;
    O* Cg = reinterpret_cast<O*>(a.C);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int p = v * THREADS + tid;
      if (p >= P) continue;
      const int nb = p / 64, l = p % 64;
      const int m = l & 15, n = n0 + 16 * nb + 4 * (l >> 4);
      if (m >= a.M) continue;
      O* dst = Cg + (size_t)m * a.N + n;
      if (a.c_vec && n + 4 <= a.N) {
        typedef O o4 __attribute__((ext_vector_type(4)));
        o4 w = {cvt_out<DT>(sum[v][0]), cvt_out<DT>(sum[v][1]), cvt_out<DT>(sum[v][2]),
                cvt_out<DT>(sum[v][3])};
        *reinterpret_cast<o4*>(dst) = w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) dst[e] = cvt_out<DT>(sum[v][e]);
      }
    }
  };
  if (a.dtype_c == DT_F16) store(std::integral_constant<int, DT_F16>{});
  else if (a.dtype_c == DT_BF16) store(std::integral_constant<int, DT_BF16>{});
  else store(std::integral_constant<int, DT_F32>{});
}

// ================================================================= instantiation table

using LaunchFn = hipError_t (*)(const Plan&, const KArgs&, hipStream_t);

template <class T, bool A_KC, bool B_KC, bool U4B, int MT_M, int MT_N, int WM, int WN, int LROWS,
          int PP, int DTL, int MI>
hipError_t launch_tile(const Plan& p, const KArgs& a, hipStream_t s) {
  using Cfg = TileCfg<T, A_KC, B_KC, U4B, MT_M, MT_N, WM, WN, LROWS, DTL, MI>;
  dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, (unsigned)p.grid_z);
  hipLaunchKernelGGL((gemm_tile_kernel<T, A_KC, B_KC, U4B, MT_M, MT_N, WM, WN, LROWS, PP, DTL, MI>),
                     grid, dim3(Cfg::THREADS), 0, s, a);
  return hipGetLastError();
}

template <class T, bool U4B, int NB, int W, int U>
hipError_t launch_skinny(const Plan& p, const KArgs& a, hipStream_t s) {
  dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, (unsigned)p.grid_z);
  hipLaunchKernelGGL((gemm_skinny_kernel<T, U4B, NB, W, U>), grid, dim3(W * 64), 0, s, a);
  return hipGetLastError();
}

template <class T> constexpr int dt_code() {
  return std::is_same<T, F16T>::value ? DT_F16 : (std::is_same<T, F8T>::value ? DT_F8 : DT_BF16);
}

struct Variant {
  VariantInfo info;
  LaunchFn fn;
};

#define TILE_XM(T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, PP, DTL, MI)                       \
  Variant{VariantInfo{KERNEL_TILE, dt_code<T>(), (U4) ? DT_U4 : dt_code<T>(), (AKC) ? 0 : 1,  \
                      (BKC) ? 1 : 0, MTM, MTN,                                               \
                      TileCfg<T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, DTL, MI>::BK, (WM) * (WN), 1, PERM, \
                      TileCfg<T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, DTL, MI>::lds_alloc(PP),  \
                      TileCfg<T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, DTL, MI>::NSETS, 1, PP,   \
                      (TileCfg<T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, DTL, MI>::A_DTL ? 1 : 0) | \
                      (TileCfg<T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, DTL, MI>::B_DTL ? 2 : 0) | \
                      (TileCfg<T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, DTL, MI>::A_TR ? 4 : 0) |  \
                      (TileCfg<T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, DTL, MI>::B_TR ? 8 : 0), MI}, \
          &launch_tile<T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, PP, DTL, MI>}
#define TILE_X(T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, PP, DTL) TILE_XM(T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, PP, DTL, 32)
#define TILE_PP(T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, PP) TILE_X(T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, PP, 0)
#define TILE(T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM) TILE_X(T, AKC, BKC, U4, MTM, MTN, WM, WN, PERM, false, 0)
#define TILE_DTL(T, AKC, BKC, U4, MTM, MTN, WM, WN) TILE_X(T, AKC, BKC, U4, MTM, MTN, WM, WN, true, false, 1)
#define TILE_DTLTR(T, AKC, BKC, U4, MTM, MTN, WM, WN) TILE_X(T, AKC, BKC, U4, MTM, MTN, WM, WN, true, false, 2)

#define TILE_LAYOUTS(T, MTM, MTN, WM, WN)                                                    \
  TILE(T, true, true, false, MTM, MTN, WM, WN, true),                                      \
  TILE(T, true, false, false, MTM, MTN, WM, WN, true),                                     \
  TILE(T, false, true, false, MTM, MTN, WM, WN, true),                                     \
  TILE(T, false, false, false, MTM, MTN, WM, WN, true)

// Layouts with at least one K-contiguous operand, direct-to-LDS loads for those.
#define TILE_LAYOUTS_DTL(T, MTM, MTN, WM, WN)                                                \
  TILE_DTL(T, true, true, false, MTM, MTN, WM, WN),                                        \
  TILE_DTL(T, true, false, false, MTM, MTN, WM, WN),                                       \
  TILE_DTL(T, false, true, false, MTM, MTN, WM, WN)

// Layouts with at least one transposed operand, every operand loaded straight into LDS and
// the transposed ones transposed by the LDS reads.
#define TILE_LAYOUTS_DTLTR(T, MTM, MTN, WM, WN)                                              \
  TILE_DTLTR(T, true, false, false, MTM, MTN, WM, WN),                                     \
  TILE_DTLTR(T, false, true, false, MTM, MTN, WM, WN),                                     \
  TILE_DTLTR(T, false, false, false, MTM, MTN, WM, WN)

// Layouts with at least one K-contiguous operand: the ping-pong schedule with direct-to-LDS
// loads for those operands.
#define TILE_LAYOUTS_PPDTL(T, MTM, MTN, WM, WN)                                              \
  TILE_X(T, true, true, false, MTM, MTN, WM, WN, true, true, 1),                           \
  TILE_X(T, true, false, false, MTM, MTN, WM, WN, true, true, 1),                          \
  TILE_X(T, false, true, false, MTM, MTN, WM, WN, true, true, 1)

// Layouts with at least one transposed operand: the ping-pong schedule with every operand
// loaded straight into LDS, the transposed ones in global order, transposed by the LDS reads.
#define TILE_LAYOUTS_PPTR(T, MTM, MTN, WM, WN)                                               \
  TILE_X(T, true, false, false, MTM, MTN, WM, WN, true, true, 2),                          \
  TILE_X(T, false, true, false, MTM, MTN, WM, WN, true, true, 2),                          \
  TILE_X(T, false, false, false, MTM, MTN, WM, WN, true, true, 2)

// Every layout on schedule 2 (4 waves, every operand straight into LDS, the transposed
// ones transposed by the LDS reads, one barrier per step after sub-step 2).
#define TILE_LAYOUTS_W4(T, MTM, MTN)                                                         \
  TILE_X(T, true, true, false, MTM, MTN, 2, 2, true, 2, 1),                                \
  TILE_X(T, false, true, false, MTM, MTN, 2, 2, true, 2, 2),                               \
  TILE_X(T, true, false, false, MTM, MTN, 2, 2, true, 2, 2),                               \
  TILE_X(T, false, false, false, MTM, MTN, 2, 2, true, 2, 2)

// Every layout on the ping-pong schedule with 16x16x32 blocks and every operand straight
// into LDS (K-contiguous ones in rows, transposed ones in 64-wide K-row segments for the
// transposing reads): 8-wave tiles whose wave tiles are not whole 32x32 blocks.
#define TILE_LAYOUTS_PP16(T, MTM, MTN)                                                       \
  TILE_XM(T, true, true, false, MTM, MTN, 2, 4, true, 1, 1, 16),                           \
  TILE_XM(T, false, true, false, MTM, MTN, 2, 4, true, 1, 2, 16),                          \
  TILE_XM(T, true, false, false, MTM, MTN, 2, 4, true, 1, 2, 16),                          \
  TILE_XM(T, false, false, false, MTM, MTN, 2, 4, true, 1, 2, 16)

#define TILE_LAYOUTS_PP(T, MTM, MTN, WM, WN)                                                 \
  TILE_PP(T, true, true, false, MTM, MTN, WM, WN, true, true),                             \
  TILE_PP(T, true, false, false, MTM, MTN, WM, WN, true, true),                            \
  TILE_PP(T, false, true, false, MTM, MTN, WM, WN, true, true),                            \
  TILE_PP(T, false, false, false, MTM, MTN, WM, WN, true, true)

#define SKINNY(T, U4, NB, W, U, SLOTS)                                                       \
  Variant{VariantInfo{KERNEL_SKINNY, dt_code<T>(), (U4) ? DT_U4 : dt_code<T>(), 0, 1, 16,     \
                      16 * (NB), (U4) ? 128 : 64, W, W, 0, 0, U, SLOTS, 0, 0, 16},           \
          &launch_skinny<T, U4, NB, W, U>}


// Instantiation tables, one per translation unit.
int variants_f16(const Variant** out);
int variants_bf16(const Variant** out);
int variants_f8(const Variant** out);
int variants_misc(const Variant** out);

}  // namespace dg
