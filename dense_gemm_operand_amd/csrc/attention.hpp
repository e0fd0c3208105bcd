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
// Workgroup: 8 waves, 256 query rows (32 per wave); keys in units of 64. Software
// pipeline, step j (one barrier per step):
//   1. S(j+1) = Q K(j+1)^T with v_mfma_f32_32x32x16 (Q fragments stay in registers, K
//      fragments are 16-byte reads of [key][d] LDS rows), interleaved with
//   2. the online softmax of S(j) (computed in step j-1) in the exp2 domain: running row
//      maximum, partial row sums per lane, the output rescaled by exp2(m_old - m_new);
//   3. O += P(j) V(j), with P taken straight from the score registers: a lane's score
//      layout (keys 8g + 4*(lane/32) + c of its query row) is used as the K order of the
//      P fragment, and V's LDS rows store each group of 16 keys in the matching order
//      (4-key groups 0, 2, 1, 3), so a V fragment is one 16-byte read;
//   4. LDS stores of K(j+2) and V(j+1) (loaded in step j-1: waves 0-3 load and transpose
//      V, waves 4-7 load K, so every SIMD holds one of each), then the loads of K(j+3) and
//      V(j+2).
// K and V each use two LDS stages; a stage is rewritten one barrier after its last read.
// The last step applies the key mask (keys past Sk get no weight) and computes no S(j+1).
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

// acc + x.lo + x.hi for a packed pair of 16-bit values (v_dot2 with (1, 1): the products
// are exact and the sum is taken in fp32).
template <class T>
__device__ __forceinline__ float sum2(uint32_t x, float acc);
template <>
__device__ __forceinline__ float sum2<F16T>(uint32_t x, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), one, acc, false);
}
template <>
__device__ __forceinline__ float sum2<BF16T>(uint32_t x, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
}

// NEG: the scale is negative, so the largest scaled score comes from the smallest score.
template <class T, bool NEG>
__global__ __launch_bounds__(512) void attn_fwd_kernel(AttnArgs a) {
  constexpr int D = 128, BM = 256, BN = 64;
  constexpr int KPITCH = 2 * D + 16;     // K rows [key][d]: 256 B + pad
  constexpr int VPITCH = 2 * BN + 16;    // V rows [d][key]: 128 B + pad
  constexpr int KT = BN * KPITCH, VT = D * VPITCH;
  constexpr RowPerm PV = RowPerm{64, 8}; // V's d rows
  constexpr int SMEM = 2 * KT + 2 * VT;
  static_assert(BM * KPITCH <= SMEM, "the output tile is staged in the same LDS");
  __shared__ __attribute__((aligned(16))) char lds[SMEM];   // K stage 0, 1, V stage 0, 1
  auto kst = [&](int s) { return lds + s * KT; };
  auto vst = [&](int s) { return lds + 2 * KT + s * VT; };

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

  // Loads of one key unit. Waves 0-3 (x = tid): V block (kh2, v, rest) = (x % 2, x / 2 % 16,
  // x / 32): keys 4kg + j, kg = 4(rest / 2) + 2 kh2 + rest % 2, of d vector 8v. Waves 4-7
  // (x = tid - 256): K chunk c = y % 16 of key row y / 16, y = 256 i + x (16 lanes per
  // 256-byte row).
  const bool v_role = wave < 4;
  const int x = v_role ? tid : tid - 256;
  const size_t kv0 = (size_t)bh * a.Sk;
  const int vkh = x & 1, vv = (x >> 1) & 15, vrest = x >> 5;
  const int vkg = 4 * (vrest >> 1) + 2 * vkh + (vrest & 1);
  u32x4 rg[4];
  auto load_v = [&](int unit) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = unit * BN + 4 * vkg + j;
      rg[j] = ld128(rV, key < a.Sk ? (uint32_t)((kv0 + key) * D + 8 * vv) * 2u : kOOB);
    }
  };
  auto load_k = [&](int unit) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int y = 256 * i + x, key = unit * BN + (y >> 4);
      rg[i] = ld128(rK, key < a.Sk ? (uint32_t)((kv0 + key) * D + 8 * (y & 15)) * 2u : kOOB);
    }
  };
  // V transposed: element e of the d vector (four keys, 8 bytes) to row inv(8v + e) at
  // byte 16 rest + 8 kh2, which puts the 4-key groups of every 16 keys in order 0, 2, 1, 3.
  auto store_v = [&](int s) {
    char* vb = vst(s);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<u32x2*>(vb + PV.inv(8 * vv + e) * VPITCH + 16 * vrest + 8 * vkh) = transpose_row4(rg, e);
  };
  auto store_k = [&](int s) {
    char* kb = kst(s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int y = 256 * i + x;
      *reinterpret_cast<u32x4*>(kb + (y >> 4) * KPITCH + 16 * (y & 15)) = rg[i];
    }
  };

  // S = Q K^T for the 64 keys in K stage s: two 32-key blocks.
  auto scores = [&](auto ST_, f32x16 (&S)[2]) {
    const char* kb = kst(decltype(ST_)::value);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) S[b][e] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kb + (32 * b + r32) * KPITCH + 16 * (2 * k + kh));
        S[b] = mfma32x32x16<T>(kf, q[k], S[b]);
      }
  };

  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  // m_run: the row's reference maximum (scaled, log2 domain); l_run: this lane's share of
  // the row sum of the weights relative to it.
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;
  constexpr float MASKED = NEG ? INFINITY : -INFINITY;

  // Row maximum of S (scaled): the lane's 32 scores and its partner lane's (lane ^ 32).
  // Masked scores (keys past Sk) are set so that they never win.
  auto row_max = [&](f32x16 (&S)[2], int key0, auto MASK_) {
    if constexpr (decltype(MASK_)::value) {
      const int klim = a.Sk - key0 - 4 * kh;   // element (b, e) is valid iff its offset < klim
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * b + 8 * (e >> 2) + (e & 3) >= klim) S[b][e] = MASKED;
    }
    float r = S[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) r = NEG ? fminf(r, S[b][e]) : fmaxf(r, S[b][e]);
    r = NEG ? fminf(r, __shfl_xor(r, 32)) : fmaxf(r, __shfl_xor(r, 32));
    return r * sl2;
  };

  // The reference maximum is raised only when some row's maximum exceeds it by more than
  // 8 (a factor 256): the weights exp2(s - m_run) then stay <= 256, well inside fp16, and
  // the output and sums are rescaled (64 multiplies) only in those steps. The result does
  // not depend on which reference is used (it cancels in O / l).
  auto rebase = [&](float mx) {
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
    }
  };

  // Weights of S (keys of one unit) as P fragments, their row sum (the fp16/bf16 values the
  // second product uses, added exactly in fp32 by v_dot2), then O += P V from V stage VS.
  auto weights_pv = [&](f32x16 (&S)[2], auto VS_, int key0, auto MASK_) {
    constexpr bool MASK = decltype(MASK_)::value;
    const int klim = a.Sk - key0 - 4 * kh;
    u32x4 pf[4];   // P fragment of sub-step (b, u2): the lane's scores 8u2 .. 8u2 + 7 of block b
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int e0 = 8 * u2 + 2 * w;
          float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[b][e0], sl2, -m_run));
          float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[b][e0 + 1], sl2, -m_run));
          if constexpr (MASK) {
            p0 = 32 * b + 8 * (e0 >> 2) + (e0 & 3) < klim ? p0 : 0.f;
            p1 = 32 * b + 8 * ((e0 + 1) >> 2) + ((e0 + 1) & 3) < klim ? p1 : 0.f;
          }
          pf[2 * b + u2][w] = pack2<T>(p0, p1);
          l_run = sum2<T>(pf[2 * b + u2][w], l_run);
        }
    // O += P V: sub-step i = 2b + u2 covers keys 32b + 16u2 + 0..15; the V fragment of d
    // block db is row 32db + r32, 16-byte chunk 2i + kh.
    const char* vb = vst(decltype(VS_)::value);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x4 vf = *reinterpret_cast<const u32x4*>(vb + (32 * db + r32) * VPITCH + 16 * (2 * i + kh));
        o[db] = mfma32x32x16<T>(vf, pf[i], o[db]);
      }
  };

  const int nu = (a.Sk + BN - 1) / BN;
  const bool ragged = nu * BN != a.Sk;
  // Prologue: K(0), V(0), K(1) into LDS, S(0) and its row maximum, then the loads of
  // K(2) / V(1).
  if (v_role) { load_v(0); store_v(0); } else { load_k(0); store_k(0); }
  if (!v_role) { load_k(1); store_k(1); }
  __syncthreads();
  using TRUE = std::integral_constant<bool, true>;
  using FALSE = std::integral_constant<bool, false>;
  f32x16 SA[2], SB[2];
  scores(IC<0>{}, SA);
  float mx = (ragged && nu == 1) ? row_max(SA, 0, TRUE{}) : row_max(SA, 0, FALSE{});
  if (v_role) load_v(1); else load_k(2);
  __syncthreads();   // K stage 0 is rewritten in step 0

  // Step j (S(j) in Sc, its row maximum in mx): S(j+1) into Sn, the weights of S(j) and
  // O += P(j) V(j), the row maximum of S(j+1) (masked if unit j+1 is the ragged last
  // one), the LDS stores of K(j+2) -> K stage j%2 (last read in step j-1) and V(j+1) -> V
  // stage (j+1)%2 (last read in step j-1), the loads of the step after, one barrier.
  // Written for even and odd j so that stages are compile-time.
  auto step = [&](int j, auto P_, f32x16 (&Sc)[2], f32x16 (&Sn)[2]) {
    constexpr int P = decltype(P_)::value;   // j % 2
    rebase(mx);
    scores(IC<P ^ 1>{}, Sn);
    weights_pv(Sc, IC<P>{}, j * BN, FALSE{});
    mx = (ragged && j + 2 == nu) ? row_max(Sn, (j + 1) * BN, TRUE{}) : row_max(Sn, (j + 1) * BN, FALSE{});
    if (v_role) { store_v(P ^ 1); load_v(j + 2); }
    else { store_k(P); load_k(j + 3); }
    __syncthreads();
  };
  int j = 0;
  for (; j + 2 < nu; j += 2) {
    step(j, IC<0>{}, SA, SB);
    step(j + 1, IC<1>{}, SB, SA);
  }
  // the last unit (j = nu - 1): weights and P V only (the mask leaves a full unit whole)
  auto last = [&](f32x16 (&Sc)[2], auto P_) {
    rebase(mx);
    weights_pv(Sc, P_, j * BN, TRUE{});
  };
  if (j + 1 < nu) {          // one more full step (j even), then the last unit (odd)
    step(j, IC<0>{}, SA, SB);
    ++j;
    last(SB, IC<1>{});
  } else {
    last(SA, IC<0>{});
  }
  __syncthreads();   // the output tile reuses the LDS

  // ---- epilogue: row sum of both lanes, O / l, staged by logical d, 16-byte row stores
  const float l = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l;
  using O_t = typename std::conditional<std::is_same<T, F16T>::value, _Float16, __bf16>::type;
  typedef O_t o4 __attribute__((ext_vector_type(4)));
  char* stg = lds;  // 256 rows x KPITCH bytes
  const int srow = 32 * wave + r32;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // physical d rows 32db + 8g + 4kh + c (g = 0..3) are logical fwd(32db + 4kh + c) + g
      const int d = PV.fwd(32 * db + 4 * kh + c);
      const o4 w = {(O_t)(o[db][c] * inv), (O_t)(o[db][4 + c] * inv), (O_t)(o[db][8 + c] * inv),
                    (O_t)(o[db][12 + c] * inv)};
      *reinterpret_cast<o4*>(stg + srow * KPITCH + 2 * d) = w;
    }
  __syncthreads();
  O_t* Og = reinterpret_cast<O_t*>(a.O);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int y = 512 * i + tid, row = y >> 4, c = y & 15;
    const int gq = m0 + row;
    if (gq < a.Sq)
      *reinterpret_cast<u32x4*>(Og + ((size_t)bh * a.Sq + gq) * D + 8 * c) =
          *reinterpret_cast<const u32x4*>(stg + row * KPITCH + 16 * c);
  }
}

}  // namespace dg
