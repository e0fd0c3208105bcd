// Host-side sanitizer driver: exercises the library's host code (argument checks, planner,
// plan queries, the int4 repack, the LDS permutation view, status strings, the attention
// entry's argument checks) and the CPU oracle's C functions, in a build of host.cpp and
// oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py builds
// and runs it; device code is not instrumented). No GPU is touched: plans are made with
// DGEMM_FAKE_CU_COUNT, so gemm_run stops at its device check. Exit status 0 when every check
// passed and no sanitizer fired (sanitizer reports abort the process).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../include/dattn.h"
#include "../include/dgemm.h"

extern "C" {
int oracle_decode(const void* src, int64_t n, int code, double* dst);
int oracle_encode(const double* src, int64_t n, int code, void* dst);
int oracle_logical(const double* stored, int64_t rows, int64_t cols, int col_major, double* logical);
int oracle_dequant_u4(const uint8_t* packed, const uint16_t* scales, int64_t K, int64_t N,
                      int64_t group, int zero, double* logical_kn);
int oracle_gemm_f64(const double* a, const double* b, int64_t M, int64_t N, int64_t K,
                    int64_t row_begin, int64_t row_end, double* c);
int oracle_attention_f64(const double* q, const double* k, const double* v, int64_t BH,
                         int64_t Sq, int64_t Sk, int64_t D, double scale, int64_t row_begin,
                         int64_t row_end, double* o);
}

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static void planner() {
  const int64_t sizes[] = {1, 7, 8, 16, 17, 64, 100, 128, 255, 256, 264, 1000, 3072, 4096, 28672};
  const int dts[][3] = {{GEMM_F16, GEMM_F16, GEMM_F32}, {GEMM_F16, GEMM_F16, GEMM_F16},
                        {GEMM_BF16, GEMM_BF16, GEMM_BF16}, {GEMM_F8, GEMM_F8, GEMM_F16},
                        {GEMM_F16, GEMM_U4, GEMM_F16}, {GEMM_F32, GEMM_F32, GEMM_F32}};
  const gemm_quant_t quants[] = {{128, 8, GEMM_F16, 0}, {32, 0, GEMM_F16, 0}, {48, 8, GEMM_F16, 0},
                                 {128, 16, GEMM_F16, 0}};
  int made = 0, refused = 0;
  for (int64_t M : sizes)
    for (int64_t N : {(int64_t)8, (int64_t)200, (int64_t)512, (int64_t)5120, (int64_t)8192})
      for (int64_t K : {(int64_t)64, (int64_t)136, (int64_t)1000, (int64_t)8192})
        for (int la = 0; la < 2; ++la)
          for (int lb = 0; lb < 3; ++lb)
            for (const auto& dt : dts)
              for (int sk : {0, 1, 3, 4, 16})
                for (int q = 0; q < (dt[1] == GEMM_U4 ? 4 : 1); ++q) {
                  gemm_plan_t p = reinterpret_cast<gemm_plan_t>(0x1);
                  const int st = gemm_plan(&p, M, N, K, la, lb, dt[0], dt[1], dt[2], sk,
                                           dt[1] == GEMM_U4 ? &quants[q] : nullptr);
                  if (st != GEMM_OK) {
                    CHECK(p == nullptr);
                    CHECK(st < 0 && std::strcmp(gemm_status_string(st), "unknown status") != 0);
                    ++refused;
                    continue;
                  }
                  ++made;
                  gemm_plan_info_t info;
                  CHECK(gemm_plan_query(p, &info) == GEMM_OK);
                  CHECK(info.M == M && info.N == N && info.K == K);
                  CHECK(info.grid_x * info.grid_y * info.grid_z >= 1);
                  CHECK(info.split_k >= 1 && info.split_k <= 16);
                  size_t ws = 1;
                  CHECK(gemm_workspace_size(p, &ws) == GEMM_OK);
                  CHECK((ws == 0) == (info.split_k == 1));
                  // no device was bound (fake CU count): the run stops at its device check
                  std::vector<uint8_t> buf(64);
                  void* d = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(buf.data()) + 15) & ~uintptr_t(15));
                  const int rs = gemm_run(p, d, d, d, d, ws ? d : nullptr, ws, nullptr);
                  CHECK(rs == GEMM_ERR_NO_DEVICE || rs == GEMM_ERR_WORKSPACE_TOO_SMALL);
                  CHECK(gemm_run(p, nullptr, d, d, d, nullptr, 0, nullptr) == GEMM_ERR_INVALID_ARG);
                  gemm_plan_destroy(p);
                }
  CHECK(made > 1000 && refused > 100);
  std::printf("planner: %d plans made, %d refused\n", made, refused);
  // argument errors
  gemm_plan_t p = nullptr;
  CHECK(gemm_plan(nullptr, 8, 8, 8, 0, 1, GEMM_F16, GEMM_F16, GEMM_F16, 1, nullptr) == GEMM_ERR_INVALID_ARG);
  CHECK(gemm_plan(&p, -1, 8, 8, 0, 1, GEMM_F16, GEMM_F16, GEMM_F16, 1, nullptr) == GEMM_ERR_INVALID_ARG);
  CHECK(gemm_plan(&p, 8, 8, 8, 5, 1, GEMM_F16, GEMM_F16, GEMM_F16, 1, nullptr) == GEMM_ERR_INVALID_ARG);
  CHECK(gemm_plan(&p, (int64_t)1 << 40, (int64_t)1 << 40, 8, 0, 1, GEMM_F16, GEMM_F16, GEMM_F16, 1, nullptr) == GEMM_ERR_UNSUPPORTED);
  CHECK(gemm_plan(&p, INT64_MAX, INT64_MAX, INT64_MAX, 0, 1, GEMM_F16, GEMM_F16, GEMM_F16, 0, nullptr) == GEMM_ERR_UNSUPPORTED);
  size_t ws = 0;
  CHECK(gemm_workspace_size(nullptr, &ws) == GEMM_ERR_INVALID_ARG);
  CHECK(gemm_plan_query(nullptr, nullptr) == GEMM_ERR_INVALID_ARG);
  gemm_plan_destroy(nullptr);
  for (int s = -20; s <= 2; ++s) CHECK(gemm_status_string(s) != nullptr);
}

static void repack_and_permutation() {
  const int64_t N = 128, K = 256;
  std::vector<uint8_t> codes(N * K / 2), tiled(N * K / 2);
  for (size_t i = 0; i < codes.size(); ++i) codes[i] = (uint8_t)(i * 37 + 11);
  CHECK(gemm_pack_u4_tiled(codes.data(), tiled.data(), N, K) == GEMM_OK);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < K / 128; ++g)
      CHECK(std::memcmp(&tiled[((n / 64) * (K / 128) + g) * 4096 + (n % 64) * 64],
                        &codes[n * (K / 2) + g * 64], 64) == 0);
  CHECK(gemm_pack_u4_tiled(codes.data(), tiled.data(), 100, K) == GEMM_ERR_UNSUPPORTED);
  CHECK(gemm_pack_u4_tiled(nullptr, tiled.data(), N, K) == GEMM_ERR_INVALID_ARG);
  for (int B = 1; B <= 512; ++B)
    for (int S = 1; S <= B; ++S) {
      if (B % S) {
        CHECK(gemm_lds_row_perm(B, S, 0, 0) == -1);
        continue;
      }
      for (int I = 0; I < B; ++I) {
        const int f = gemm_lds_row_perm(B, S, I, 0);
        CHECK(f >= 0 && f < B && gemm_lds_row_perm(B, S, f, 1) == I);
      }
    }
  CHECK(gemm_lds_row_perm(8, 2, 8, 0) == -1 && gemm_lds_row_perm(0, 1, 0, 0) == -1);
}

static void attention_checks() {
  std::vector<uint8_t> buf(64);
  void* d = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(buf.data()) + 15) & ~uintptr_t(15));
  CHECK(attn_fwd(nullptr, d, d, d, 1, 1, 1, 128, GEMM_F16, 1.f, nullptr) == GEMM_ERR_INVALID_ARG);
  CHECK(attn_fwd(d, d, d, d, 0, 1, 1, 128, GEMM_F16, 1.f, nullptr) == GEMM_ERR_INVALID_ARG);
  CHECK(attn_fwd(d, d, d, d, 1, 1, 1, 64, GEMM_F16, 1.f, nullptr) == GEMM_ERR_UNSUPPORTED);
  CHECK(attn_fwd(d, d, d, d, 1, 1, 1, 128, GEMM_F8, 1.f, nullptr) == GEMM_ERR_UNSUPPORTED);
  CHECK(attn_fwd(d, d, d, d, 1, 1, 1, 128, GEMM_F16, NAN, nullptr) == GEMM_ERR_INVALID_ARG);
  CHECK(attn_fwd(d, d, d, d, INT64_MAX, INT64_MAX, 1, 128, GEMM_F16, 1.f, nullptr) == GEMM_ERR_UNSUPPORTED);
  CHECK(attn_fwd(d, d, d, d, (int64_t)1 << 20, (int64_t)1 << 20, 1, 128, GEMM_F16, 1.f, nullptr) == GEMM_ERR_UNSUPPORTED);
}

static void oracle_checks() {
  // every binary16 and bfloat16 pattern decodes and re-encodes to itself (NaNs to a NaN)
  for (int code = 0; code < 2; ++code) {
    std::vector<uint16_t> bits(65536), back(65536);
    for (int i = 0; i < 65536; ++i) bits[i] = (uint16_t)i;
    std::vector<double> v(65536);
    CHECK(oracle_decode(bits.data(), 65536, code, v.data()) == 0);
    CHECK(oracle_encode(v.data(), 65536, code, back.data()) == 0);
    for (int i = 0; i < 65536; ++i) CHECK(std::isnan(v[i]) || back[i] == bits[i]);
  }
  std::vector<uint8_t> f8(256);
  std::vector<double> v8(256);
  for (int i = 0; i < 256; ++i) f8[i] = (uint8_t)i;
  CHECK(oracle_decode(f8.data(), 256, 3, v8.data()) == 0);
  CHECK(v8[0x38] == 1.0 && v8[0x7e] == 448.0 && std::isnan(v8[0x7f]));
  CHECK(oracle_decode(f8.data(), 4, 9, v8.data()) == -1);
  // a small product: logical maps, fp64 sums, a row range
  const int64_t M = 5, N = 7, K = 9;
  std::vector<double> as(M * K), bs(K * N), a(M * K), b(K * N), c(M * N);
  for (int64_t i = 0; i < M * K; ++i) as[i] = (double)(i % 7) - 3;
  for (int64_t i = 0; i < K * N; ++i) bs[i] = (double)(i % 5) - 2;
  CHECK(oracle_logical(as.data(), M, K, 1, a.data()) == 0);
  CHECK(oracle_logical(bs.data(), K, N, 0, b.data()) == 0);
  CHECK(oracle_gemm_f64(a.data(), b.data(), M, N, K, 0, M, c.data()) == 0);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double s = 0;
      for (int64_t k = 0; k < K; ++k) s += as[i + k * M] * bs[k * N + j];
      CHECK(c[i * N + j] == s);
    }
  CHECK(oracle_gemm_f64(a.data(), b.data(), M, N, K, 2, 9, c.data()) == -1);
  // int4 dequant
  std::vector<uint8_t> packed(N * 128 / 2);
  std::vector<uint16_t> sc(N);
  for (size_t i = 0; i < packed.size(); ++i) packed[i] = (uint8_t)(i * 13);
  for (int64_t n = 0; n < N; ++n) sc[n] = 0x3c00;   // 1.0
  std::vector<double> w(128 * N);
  CHECK(oracle_dequant_u4(packed.data(), sc.data(), 128, N, 128, 8, w.data()) == 0);
  for (int64_t k = 0; k < 128; ++k)
    for (int64_t n = 0; n < N; ++n) {
      const uint8_t byte = packed[n * 64 + k / 2];
      const int q = (k % 2) ? byte >> 4 : byte & 15;
      CHECK(w[k * N + n] == (double)(q - 8));
    }
  CHECK(oracle_dequant_u4(packed.data(), sc.data(), 127, N, 128, 8, w.data()) == -1);
  // attention: one key gives its value row
  const int64_t BH = 2, Sq = 3, Sk = 1, D = 4;
  std::vector<double> q(BH * Sq * D, 0.5), kk(BH * Sk * D, 0.25), vv(BH * Sk * D), o(BH * Sq * D);
  for (int64_t i = 0; i < BH * Sk * D; ++i) vv[i] = (double)i;
  CHECK(oracle_attention_f64(q.data(), kk.data(), vv.data(), BH, Sq, Sk, D, 1.0, 0, BH * Sq, o.data()) == 0);
  for (int64_t r = 0; r < BH * Sq; ++r)
    for (int64_t d = 0; d < D; ++d) CHECK(o[r * D + d] == vv[(r / Sq) * D + d]);
  CHECK(oracle_attention_f64(q.data(), kk.data(), vv.data(), BH, Sq, 0, D, 1.0, 0, 1, o.data()) == -1);
}

int main() {
  setenv("DGEMM_FAKE_CU_COUNT", "256", 1);
  planner();
  repack_and_permutation();
  attention_checks();
  oracle_checks();
  std::printf("%s: %d failed checks\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
