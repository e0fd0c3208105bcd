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
// Workgroup: 8 waves, 256 query rows (32 per wave); keys in units of 64. Per unit k, two
// phases, each ending with a workgroup barrier:
//   X(k): the online softmax of S(k) in the exp2 domain (running row maximum, partial row
//         sums per lane, the output rescaled only when the maximum grows by more than 8),
//         producing the P fragments: P is taken straight from the score registers (a
//         lane's score layout, keys 8g + 4*(lane/32) + c of its query row, is used as the
//         K order of the P fragment, and V's LDS rows store each group of 16 keys in the
//         matching order, 4-key groups 0, 2, 1, 3, so a V fragment is one 16-byte read);
//   M(k): S(k+1) = Q K(k+1)^T and O += P(k) V(k) with v_mfma_f32_32x32x16 (Q fragments
//         stay in registers, K and V fragments are 16-byte LDS reads), then this wave
//         group's half of the LDS stores of K(k+2) and V(k+1) and of the loads after them.
// The two wave groups (waves 0-3 and 4-7; waves w and w + 4 share a SIMD) run one phase
// apart, so on every SIMD one wave's softmax (vector ALU) runs beside the other wave's
// matrix-core phase. K and V each use two LDS stages (lifetimes are stated with the
// schedule below). The last unit applies the key mask (keys past Sk get no weight).
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
  const int grp = wave >> 2;   // waves w and w + 4 share a SIMD: one of each group

  // Workgroup -> (slice, query block), XCD-aware: consecutive ids go round-robin over the
  // 8 XCDs, so each XCD is given a contiguous range and the query blocks of one slice
  // (which read the same K and V) share an L2.
  const int total = a.BH * a.q_blocks;
  int t = blockIdx.x;
  if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;
  const int bh = t / a.q_blocks, qb = t % a.q_blocks;
  const int m0 = qb * BM;

  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(a.Q, a.bytesQ);
  // K and V of this slice only: a key at or past Sk starts at or past num_records, where
  // buffer loads return zeros, so the loads need no bounds arithmetic.
  const size_t slice = (size_t)bh * a.Sk * D * 2;
  const uint32_t slice_bytes = (uint32_t)a.Sk * D * 2;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(static_cast<const char*>(a.K) + slice, slice_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(static_cast<const char*>(a.V) + slice, slice_bytes);

  // The wave's Q fragments: lane row r32 of its 32 rows, d = 16s + 8kh + 0..7.
  u32x4 q[8];
  {
    const int row = m0 + 32 * wave + r32;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      q[s] = ld128(rQ, row < a.Sq ? (uint32_t)(((size_t)bh * a.Sq + row) * D + 16 * s + 8 * kh) * 2u : kOOB);
  }

  // Each group moves half of every K and V unit: in a group, waves 0-1 (y = 0..127) take
  // V blocks, waves 2-3 K chunks. V block z = 128 grp + y: (kh2, v, rest) = (z % 2,
  // z / 2 % 16, z / 32): keys 4kg + j, kg = 4(rest / 2) + 2 kh2 + rest % 2, of d vector 8v.
  // K: chunks 512 grp + 128 i + y' (i = 0..3, y' = 0..127): chunk c % 16 of key row c / 16.
  const int gw = wave & 3;
  const bool v_role = gw < 2;
  const int y = (gw & 1) * 64 + lane;
  const int vz = 128 * grp + y;
  const int vkh = vz & 1, vv = (vz >> 1) & 15, vrest = vz >> 5;
  const int vkg = 4 * (vrest >> 1) + 2 * vkh + (vrest & 1);
  // byte offsets within the slice at unit 0 (a unit is BN * D * 2 = 16 KiB further)
  const uint32_t voff = (uint32_t)(4 * vkg * D + 8 * vv) * 2u;   // + 256 j
  const int kc0 = 512 * grp + y;                                  // + 128 i
  const uint32_t koff = (uint32_t)((kc0 >> 4) * D + 8 * (kc0 & 15)) * 2u;   // + 2048 i
  u32x4 rg[4];
  auto load_share = [&](int unit_k, int unit_v) {
    if (v_role) {
      const uint32_t u = (uint32_t)unit_v * (BN * D * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) rg[j] = ld128(rV, voff + u + 256u * j);
    } else {
      const uint32_t u = (uint32_t)unit_k * (BN * D * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) rg[i] = ld128(rK, koff + u + 2048u * i);
    }
  };
  // V transposed: element e of the d vector (four keys, 8 bytes) to row inv(8v + e) at
  // byte 16 rest + 8 kh2, which puts the 4-key groups of every 16 keys in order 0, 2, 1, 3.
  auto store_share = [&](int ks, int vs) {
    if (v_role) {
      char* vb = vst(vs);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<u32x2*>(vb + PV.inv(8 * vv + e) * VPITCH + 16 * vrest + 8 * vkh) = transpose_row4(rg, e);
    } else {
      char* kb = kst(ks);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = kc0 + 128 * i;
        *reinterpret_cast<u32x4*>(kb + (c >> 4) * KPITCH + 16 * (c & 15)) = rg[i];
      }
    }
  };

  f32x16 S[2];   // scores of one unit (two 32-key blocks)
  u32x4 pf[4];   // P fragments of that unit
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

  // The matrix-core phase issues the multiplies of S(k+1) and of P(k) V(k) alternately, so
  // six accumulators take turns (no multiply depends on the one just before it). The
  // fragment reads run FD multiplies ahead of their use (a ring of FD + 1 fragments) and the
  // program order is kept by scheduling fences.
  constexpr int FD = 3;
  // Multiply t of the phase: with scores, even t = 2s is S multiply s (k = s / 2, block
  // b = s % 2; fragment from K stage ks) and odd t = 2s + 1 is P V multiply s (i = s / 4,
  // d block db = s % 4; fragment from V stage vs); without, t is P V multiply t.
  auto is_s = [](int t, bool scores) { return scores && (t & 1) == 0; };
  auto op_idx = [](int t, bool scores) { return scores ? t >> 1 : t; };
  auto frag_addr = [&](int t, bool scores, int ks, int vs) -> const u32x4* {
    const int n = op_idx(t, scores);
    if (is_s(t, scores)) {
      const int k = n >> 1, b = n & 1;
      return reinterpret_cast<const u32x4*>(kst(ks) + (32 * b + r32) * KPITCH + 16 * (2 * k + kh));
    }
    const int i = n >> 2, db = n & 3;
    return reinterpret_cast<const u32x4*>(vst(vs) + (32 * db + r32) * VPITCH + 16 * (2 * i + kh));
  };
  // S(next) = Q K^T from K stage ks (if SCORES) and O += P V from V stage vs: sub-step
  // i = 2b + u2 of P V covers keys 32b + 16u2 + 0..15; the V fragment of d block db is
  // row 32db + r32, 16-byte chunk 2i + kh.
  auto mma_phase = [&](int ks, int vs, auto SCORES_) {
    constexpr bool SCORES = decltype(SCORES_)::value;
    constexpr int NT = SCORES ? 32 : 16;
    if constexpr (SCORES) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) S[b][e] = 0.f;
    }
    u32x4 ring[FD + 1];
#pragma unroll
    for (int t = 0; t < FD; ++t) ring[t % (FD + 1)] = *frag_addr(t, SCORES, ks, vs);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      if (t + FD < NT) ring[(t + FD) % (FD + 1)] = *frag_addr(t + FD, SCORES, ks, vs);
      const u32x4 f = ring[t % (FD + 1)];
      const int n = op_idx(t, SCORES);
      if (is_s(t, SCORES)) S[n & 1] = mfma32x32x16<T>(f, q[n >> 1], S[n & 1]);
      else o[n & 3] = mfma32x32x16<T>(f, pf[n >> 2], o[n & 3]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Softmax phase of a unit starting at key0: row maximum (the lane's 32 scores and its
  // partner lane's, keys past Sk left out), the reference update, the weights as P
  // fragments and their row sum (the fp16/bf16 values the second product uses, added
  // exactly in fp32 by v_dot2). The reference maximum is raised only when some row's
  // maximum exceeds it by more than 8 (a factor 256): the weights exp2(s - m_run) then stay
  // <= 256, well inside fp16, and the output and sums are rescaled (64 multiplies) only in
  // those steps. The result does not depend on the reference (it cancels in O / l).
  auto softmax = [&](int key0, auto MASK_) {
    constexpr bool MASK = decltype(MASK_)::value;
    const int klim = a.Sk - key0 - 4 * kh;   // element (b, e) is valid iff its offset < klim
    auto valid = [&](int b, int e) { return 32 * b + 8 * (e >> 2) + (e & 3) < klim; };
    float r = MASKED;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = (MASK && !valid(b, e)) ? MASKED : S[b][e];
        r = NEG ? fminf(r, v) : fmaxf(r, v);
      }
    r = NEG ? fminf(r, __shfl_xor(r, 32)) : fmaxf(r, __shfl_xor(r, 32));
    const float mx = r * sl2;   // finite: key0 is a valid key
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
            p0 = valid(b, e0) ? p0 : 0.f;
            p1 = valid(b, e0 + 1) ? p1 : 0.f;
          }
          pf[2 * b + u2][w] = pack2<T>(p0, p1);
          l_run = sum2<T>(pf[2 * b + u2][w], l_run);
        }
  };

  // Barrier between phases, fenced so that no instruction moves from one phase into the
  // next (matrix-core instructions have no memory effects and would drift across).
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Ping-pong schedule. Phases: M(-1) = S(0); then per unit k: X(k) = softmax of S(k);
  // M(k) = S(k+1) (if any) and O += P(k) V(k), this group's share of the LDS stores of
  // K(k+2) and V(k+1) (loaded in M(k-1)) and the loads of K(k+3) and V(k+2). Every phase
  // ends with a workgroup barrier; group 1 runs one barrier behind group 0, so on every
  // SIMD one wave's softmax (vector ALU) overlaps the other wave's matrix-core phase.
  // LDS lifetimes (intervals between barriers, group 0 in phase b while group 1 is in b-1):
  // K(k+1) and V(k) are read in intervals 2k+2 and 2k+3; K(m) is stored in intervals 2m-2
  // (group 0's half) and 2m-1 (group 1's), V(m) in 2m and 2m+1, i.e. after the last read of
  // the unit two earlier in the same stage and before the first read.
  const int nu = (a.Sk + BN - 1) / BN;
  using TRUE = std::integral_constant<bool, true>;
  using FALSE = std::integral_constant<bool, false>;
  // K(0) whole (each group its half), then this group's shares of K(1) and V(0).
  load_share(0, 0);
  if (!v_role) store_share(0, 0);
  load_share(1, 0);
  __syncthreads();
  if (grp == 1) __syncthreads();
  // M(-1): S(0) only (the loop below handles the V part of every unit)
  {
    const char* kb = kst(0);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) S[b][e] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        S[b] = mfma32x32x16<T>(*reinterpret_cast<const u32x4*>(kb + (32 * b + r32) * KPITCH + 16 * (2 * k + kh)),
                               q[k], S[b]);
  }
  store_share(1, 0);
  load_share(2, 1);
  phase_end();
  for (int k = 0; k + 1 < nu; ++k) {
    softmax(k * BN, FALSE{});                       // X(k)
    phase_end();
    mma_phase((k + 1) & 1, k & 1, TRUE{});           // M(k)
    store_share(k & 1, (k + 1) & 1);
    load_share(k + 3, k + 2);
    phase_end();
  }
  // the last unit: masked softmax, P V only (the mask leaves a full unit whole)
  softmax((nu - 1) * BN, TRUE{});
  phase_end();
  mma_phase(0, (nu - 1) & 1, FALSE{});
  phase_end();
  if (grp == 0) __syncthreads();

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
    const int z = 512 * i + tid, row = z >> 4, c = z & 15;
    const int gq = m0 + row;
    if (gq < a.Sq)
      *reinterpret_cast<u32x4*>(Og + ((size_t)bh * a.Sq + gq) * D + 8 * c) =
          *reinterpret_cast<const u32x4*>(stg + row * KPITCH + 16 * c);
  }
}

}  // namespace dg
