#pragma once
// Flash-attention forward for gfx950: O = softmax(scale * Q K^T) V per batch-head slice,
// head dimension D = 128, fp16 or bf16, fp32 scores and sums. Its second product P * V
// takes V as a non-K-contiguous operand: V is stored [key][d], and the reduction index of
// P * V is the key (Triton PR 5223, "Introduction": the second dot of flash attention is
// the other user of inThreadTranspose). V therefore goes through the same loader as a
// transposed GEMM operand: 128-bit loads of four key rows of an 8-element d vector per
// thread (thread rake), the v_perm_b32 transpose, and 64-bit LDS stores into
// key-contiguous rows, one per d, permuted by the 64-row, stride-8 block permutation
// (rocm-libraries PR 2487 formula) so that the stores spread over the banks.
//
// Workgroup: 8 waves, 256 query rows (32 per wave), K and V tiles of 128 keys. Per tile:
//   1. global loads of the next tile into registers (K rows and V blocks), in flight
//      during the whole tile;
//   2. for each half of 64 keys: S = Q K^T with v_mfma_f32_32x32x16 (the wave's Q
//      fragments stay in registers; K fragments are 16-byte LDS reads of [key][d] rows);
//      the online softmax in the exp2 domain (running row maximum and partial row sums
//      per lane, the output rescaled by exp2(m_old - m_new)); P * V with P taken straight
//      from the score registers: a lane's score layout (keys 8g + 4*(lane/32) + c of its
//      query row) is used as the K order of the P fragment, and V's LDS rows store each
//      group of 16 keys in the matching order (4-key groups 0, 2, 1, 3), so a V fragment
//      is one 16-byte read and no score moves between lanes;
//   3. LDS stores of the next tile (V transposed), one barrier.
// Epilogue: the two lanes of a row add their sums, O / l is rounded once to the output
// type, staged through LDS in logical d order and written as 16-byte row vectors.
#include "kernels.hpp"

namespace dg {

struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int BH, Sq, Sk;
  uint32_t bytesQ, bytesKV;
  float scale_log2;  // softmax scale times log2(e)
  int q_blocks;      // ceil(Sq / 256)
};

template <class T>
__device__ __forceinline__ uint32_t pack2(float x, float y);
template <>
__device__ __forceinline__ uint32_t pack2<F16T>(float x, float y) {
  const f16x2 v = {(_Float16)x, (_Float16)y};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ __forceinline__ uint32_t pack2<BF16T>(float x, float y) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)x, (__bf16)y};     // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

template <class T>
__global__ __launch_bounds__(512) void attn_fwd_kernel(AttnArgs a) {
  constexpr int D = 128, BM = 256, BN = 128, THREADS = 512;
  constexpr int PITCH = 2 * D + 16;      // K rows [key][d] and V rows [d][key]: 256 B + pad
  constexpr int TILE = 128 * PITCH;      // one operand tile (BN == D == 128 rows)
  constexpr RowPerm PV = RowPerm{64, 8}; // V's d rows
  static_assert(BN == D, "K and V tiles share the row count");
  __shared__ __attribute__((aligned(16))) char lds[2 * 2 * TILE];   // [stage][K, V]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, kh = lane >> 5;

  // Workgroup -> (slice, query block), XCD-aware: consecutive ids go round-robin over the
  // 8 XCDs, so each XCD is given a contiguous range and the query blocks of one slice
  // (which read the same K and V) share an L2.
  const int total = a.BH * a.q_blocks;
  int t = blockIdx.x;
  if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;
  const int bh = t / a.q_blocks, qb = t % a.q_blocks;
  const int m0 = qb * BM;

  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(a.Q, a.bytesQ);
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(a.K, a.bytesKV);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(a.V, a.bytesKV);

  // The wave's Q fragments: lane row r32 of its 32 rows, d = 16s + 8kh + 0..7.
  u32x4 q[8];
  {
    const int row = m0 + 32 * wave + r32;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      q[s] = ld128(rQ, row < a.Sq ? (uint32_t)(((size_t)bh * a.Sq + row) * D + 16 * s + 8 * kh) * 2u : kOOB);
  }

  // Loads of one tile. K: chunk c = x % 16 of key row x / 16, x = 512 i + tid (16 lanes per
  // 256-byte row). V: block (kh2, v, rest) = (tid % 2, tid / 2 % 16, tid / 32): keys
  // 4kg + j, kg = 4(rest / 2) + 2 kh2 + rest % 2, of d vector 8v.
  const size_t kv0 = (size_t)bh * a.Sk;
  const int vkh = tid & 1, vv = (tid >> 1) & 15, vrest = tid >> 5;
  const int vkg = 4 * (vrest >> 1) + 2 * vkh + (vrest & 1);
  u32x4 rk[4], rv[4];
  auto load_tile = [&](int it) {
    const int key0 = it * BN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 512 * i + tid, key = key0 + (x >> 4);
      rk[i] = ld128(rK, key < a.Sk ? (uint32_t)((kv0 + key) * D + 8 * (x & 15)) * 2u : kOOB);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = key0 + 4 * vkg + j;
      rv[j] = ld128(rV, key < a.Sk ? (uint32_t)((kv0 + key) * D + 8 * vv) * 2u : kOOB);
    }
  };
  // LDS stores of the loaded tile into stage `st`: K rows as loaded; V transposed, element
  // e of the d vector (four keys, 8 bytes) to row inv(8v + e) at byte 16 rest + 8 kh2, which
  // puts the 4-key groups of every 16 keys in the order 0, 2, 1, 3.
  auto store_tile = [&](int st) {
    char* kb = lds + st * 2 * TILE;
    char* vb = kb + TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 512 * i + tid;
      *reinterpret_cast<u32x4*>(kb + (x >> 4) * PITCH + 16 * (x & 15)) = rk[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<u32x2*>(vb + PV.inv(8 * vv + e) * PITCH + 16 * vrest + 8 * vkh) = transpose_row4(rv, e);
  };

  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nt = (a.Sk + BN - 1) / BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < nt; ++it) {
    const int st = it & 1;
    const char* kb = lds + st * 2 * TILE;
    const char* vb = kb + TILE;
    load_tile(it + 1);   // past the last tile every offset is out of range: zeros
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // ---- S = Q K^T for keys 64h .. 64h + 63 of the tile (two 32-key blocks)
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[b][e] = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(kb + (64 * h + 32 * b + r32) * PITCH + 16 * (2 * k + kh));
          s[b] = mfma32x32x16<T>(kf, q[k], s[b]);
        }
      }
      // ---- online softmax (log2 domain); lane holds keys 8g + 4kh + c of block b
      const int key_h = it * BN + 64 * h;
      float mloc = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = s[b][e] * a.scale_log2;
          if (key_h + 64 > a.Sk) {   // last tile only: keys past Sk get no weight
            const int key = key_h + 32 * b + 8 * (e >> 2) + 4 * kh + (e & 3);
            if (key >= a.Sk) x = -INFINITY;
          }
          s[b][e] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(s[b][e] - m_new);
          s[b][e] = p;
          lsum += p;
        }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
      // ---- O += P V: sub-step (b, u2) covers keys 64h + 32b + 16u2 + 0..15; the P fragment
      // is the lane's scores 8u2 .. 8u2 + 7 of block b, and the V fragment of d block db is
      // row 32db + r32, 16-byte chunk 2(4h + 2b + u2) + kh.
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
          u32x4 pf;
#pragma unroll
          for (int w = 0; w < 4; ++w) pf[w] = pack2<T>(s[b][8 * u2 + 2 * w], s[b][8 * u2 + 2 * w + 1]);
          const int chunk = 2 * (4 * h + 2 * b + u2) + kh;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const u32x4 vf = *reinterpret_cast<const u32x4*>(vb + (32 * db + r32) * PITCH + 16 * chunk);
            o[db] = mfma32x32x16<T>(vf, pf, o[db]);
          }
        }
      }
    }
    store_tile(st ^ 1);  // stage st^1 was last read in the previous tile, before its barrier
    __syncthreads();
  }

  // ---- epilogue: row sum of both lanes, O / l, staged by logical d, 16-byte row stores
  const float l = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l;
  using O_t = typename std::conditional<std::is_same<T, F16T>::value, _Float16, __bf16>::type;
  typedef O_t o4 __attribute__((ext_vector_type(4)));
  char* stg = lds;  // 256 rows x PITCH bytes
  const int srow = 32 * wave + r32;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // physical d rows 32db + 8g + 4kh + c (g = 0..3) are logical fwd(32db + 4kh + c) + g
      const int d = PV.fwd(32 * db + 4 * kh + c);
      const o4 w = {(O_t)(o[db][c] * inv), (O_t)(o[db][4 + c] * inv), (O_t)(o[db][8 + c] * inv),
                    (O_t)(o[db][12 + c] * inv)};
      *reinterpret_cast<o4*>(stg + srow * PITCH + 2 * d) = w;
    }
  __syncthreads();
  O_t* Og = reinterpret_cast<O_t*>(a.O);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int x = 512 * i + tid, row = x >> 4, c = x & 15;
    const int gq = m0 + row;
    if (gq < a.Sq)
      *reinterpret_cast<u32x4*>(Og + ((size_t)bh * a.Sq + gq) * D + 8 * c) =
          *reinterpret_cast<const u32x4*>(stg + row * PITCH + 16 * c);
  }
}

}  // namespace dg
