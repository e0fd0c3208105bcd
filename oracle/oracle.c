/*
 * CPU oracle for C = A * B with operands that may be stored row- or column-major, and for
 * the attention forward product whose second multiply takes a non-K-contiguous V.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, links or includes this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no header, helper, table or constant with the HIP path.
 *
 * What it computes is the plain definition of the product that every page's kernel
 * reaches up to summation order (a non-TN operand GEMM, Triton PR 5223 "Feature
 * description"; a split-K GEMM, BitBLAS PR 268 "SplitK Infer"; a dequantised-weight
 * GEMM, BitBLAS PR 268, dequantize layout example):
 *   1. decode every stored 16-bit value to fp64 (exact for binary16 and bfloat16);
 *   2. map stored positions to logical positions (row- or column-major);
 *   3. for an int4 weight operand, w = round_fp16((q - zero) * s[k / group][n]);
 *   4. c(i,j) = sum_k a(i,k) * b(k,j), a plain loop accumulating in fp64;
 *   5. round c once to the output format, round-to-nearest-even.
 * Split-K, tiling, LDS layouts and permutations are tactics that do not change this
 * definition, so none of them appears here.
 *
 * Format codes used by this file only: 0 = binary16, 1 = bfloat16, 2 = binary32,
 * 3 = 8-bit floating point E4M3 in the OCP convention (the fp8 operand format of gfx950's
 * matrix cores): sign, 4 exponent bits with bias 7, 3 fraction bits; exponent 0 is the
 * subnormal binade; there is no infinity, and only S.1111.111 is NaN, so the top
 * exponent is an ordinary binade reaching 448.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Parameters of an IEEE-style binary format with implicit leading bit. */
typedef struct {
  int mant_bits; /* stored fraction bits */
  int exp_bits;  /* exponent field width */
} fmt_t;

static int fmt_of(int code, fmt_t* f) {
  switch (code) {
    case 0: f->mant_bits = 10; f->exp_bits = 5; return 0;  /* binary16 */
    case 1: f->mant_bits = 7; f->exp_bits = 8; return 0;   /* bfloat16 */
    case 2: f->mant_bits = 23; f->exp_bits = 8; return 0;  /* binary32 */
    default: return -1;
  }
}

/* Decode one value of format f from its bit pattern, straight from the IEEE definition:
 * (-1)^s * 2^(e - bias) * 1.m for normal numbers, 2^(1 - bias) * 0.m for subnormals. */
static double decode_bits(uint32_t bits, fmt_t f) {
  const int bias = (1 << (f.exp_bits - 1)) - 1;
  const uint32_t mant_mask = (1u << f.mant_bits) - 1u;
  const uint32_t exp_mask = (1u << f.exp_bits) - 1u;
  const uint32_t sign = (bits >> (f.mant_bits + f.exp_bits)) & 1u;
  const uint32_t e = (bits >> f.mant_bits) & exp_mask;
  const uint32_t m = bits & mant_mask;
  double v;
  if (e == exp_mask) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (e == 0) {
    v = ldexp((double)m, 1 - bias - f.mant_bits);
  } else {
    v = ldexp((double)(m | (1u << f.mant_bits)), (int)e - bias - f.mant_bits);
  }
  return sign ? -v : v;
}

/* Encode x into format f with one round-to-nearest-even step.
 * The value is scaled by the quantum (spacing of representable numbers at its binade,
 * or the subnormal spacing) so that rint() performs the single rounding; the scaling is
 * by a power of two and therefore exact in fp64. Overflow gives infinity. */
static uint32_t encode_bits(double x, fmt_t f) {
  const int bias = (1 << (f.exp_bits - 1)) - 1;
  const uint32_t exp_mask = (1u << f.exp_bits) - 1u;
  const int total = f.mant_bits + f.exp_bits;
  const uint32_t sign = signbit(x) ? (1u << total) : 0u;
  if (isnan(x)) return sign | (exp_mask << f.mant_bits) | (1u << (f.mant_bits - 1));
  double a = fabs(x);
  const int emin = 1 - bias;                 /* exponent of the smallest normal */
  const int emax = bias;                     /* exponent of the largest finite */
  if (isinf(a)) return sign | (exp_mask << f.mant_bits);
  if (a == 0.0) return sign;
  int e2;
  (void)frexp(a, &e2);                       /* a = g * 2^e2, g in [0.5, 1) */
  int E = e2 - 1;                            /* a = 1.xxx * 2^E */
  int qexp = (E < emin ? emin : E) - f.mant_bits;
  double n = rint(ldexp(a, -qexp));          /* integer multiple of the quantum, RNE */
  double r = ldexp(n, qexp);                 /* rounded magnitude */
  if (r == 0.0) return sign;
  (void)frexp(r, &e2);
  E = e2 - 1;
  if (E > emax) return sign | (exp_mask << f.mant_bits);  /* rounded past the largest finite */
  if (E < emin) {                            /* subnormal: field 0, fraction = r / 2^(emin - mant) */
    uint32_t m = (uint32_t)ldexp(r, f.mant_bits - emin);
    return sign | m;
  }
  uint32_t m = (uint32_t)(ldexp(r, f.mant_bits - E) - ldexp(1.0, f.mant_bits));
  return sign | ((uint32_t)(E + bias) << f.mant_bits) | m;
}

/* One E4M3 (OCP) value from its byte, from the format's definition above. */
static double decode_e4m3(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexp((double)m, -6 - 3);          /* 0.m * 2^(1 - 7) */
  else v = ldexp((double)(8 + m), e - 7 - 3);             /* 1.m * 2^(e - 7) */
  return s ? -v : v;
}

/* Decode n stored values of format `code` (16-bit codes read uint16, binary32 reads
 * uint32, E4M3 reads bytes). */
int oracle_decode(const void* src, int64_t n, int code, double* dst) {
  if (code == 3) {
    const uint8_t* s = (const uint8_t*)src;
    for (int64_t i = 0; i < n; ++i) dst[i] = decode_e4m3(s[i]);
    return 0;
  }
  fmt_t f;
  if (fmt_of(code, &f)) return -1;
  if (code == 2) {
    const uint32_t* s = (const uint32_t*)src;
    for (int64_t i = 0; i < n; ++i) dst[i] = decode_bits(s[i], f);
  } else {
    const uint16_t* s = (const uint16_t*)src;
    for (int64_t i = 0; i < n; ++i) dst[i] = decode_bits(s[i], f);
  }
  return 0;
}

/* Round n fp64 values once (RNE) to format `code` and store the bit patterns. */
int oracle_encode(const double* src, int64_t n, int code, void* dst) {
  fmt_t f;
  if (fmt_of(code, &f)) return -1;
  if (code == 2) {
    uint32_t* d = (uint32_t*)dst;
    for (int64_t i = 0; i < n; ++i) d[i] = encode_bits(src[i], f);
  } else {
    uint16_t* d = (uint16_t*)dst;
    for (int64_t i = 0; i < n; ++i) d[i] = (uint16_t)encode_bits(src[i], f);
  }
  return 0;
}

/* Logical rows x cols matrix (row-major out) from stored data.
 * Row-major storage: element (r, c) at stored[r * cols + c].
 * Column-major storage: element (r, c) at stored[r + c * rows]. */
int oracle_logical(const double* stored, int64_t rows, int64_t cols, int col_major,
                   double* logical) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      logical[r * cols + c] = col_major ? stored[r + c * rows] : stored[r * cols + c];
  return 0;
}

/* Logical K x N weight matrix from 4-bit codes packed two per byte along K.
 * The code of (k, n) sits in byte n * (K / 2) + k / 2: the low nibble holds even k,
 * the high nibble odd k. Scales are binary16, one per group of `group` consecutive k
 * and per column: s[(k / group) * N + n]. Each weight is (q - zero) * s rounded once to
 * binary16 (q - zero is a small integer and the product is exact in fp64, so rounding
 * the fp64 product equals a correctly rounded binary16 multiply). */
int oracle_dequant_u4(const uint8_t* packed, const uint16_t* scales, int64_t K, int64_t N,
                      int64_t group, int zero, double* logical_kn) {
  fmt_t h;
  fmt_of(0, &h);
  if (K % 2 || group <= 0 || K % group) return -1;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      uint8_t byte = packed[n * (K / 2) + k / 2];
      int q = (k % 2 == 0) ? (byte & 0xF) : ((byte >> 4) & 0xF);
      double s = decode_bits(scales[(k / group) * N + n], h);
      double w = decode_bits(encode_bits((double)(q - zero) * s, h), h);
      logical_kn[k * N + n] = w;
    }
  }
  return 0;
}

/* c(i, j) = sum_{k=0}^{K-1} a(i, k) * b(k, j) in fp64 for rows i in [row_begin, row_end).
 * a is M x K row-major, b is K x N row-major, c is (row_end - row_begin) x N row-major.
 * Loop order i, k, j; rows are spread over OpenMP threads. */
int oracle_gemm_f64(const double* a, const double* b, int64_t M, int64_t N, int64_t K,
                    int64_t row_begin, int64_t row_end, double* c) {
  if (row_begin < 0 || row_end > M || row_begin > row_end) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = row_begin; i < row_end; ++i) {
    double* ci = c + (i - row_begin) * N;
    for (int64_t j = 0; j < N; ++j) ci[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double aik = a[i * K + k];
      const double* bk = b + k * N;
      for (int64_t j = 0; j < N; ++j) ci[j] += aik * bk[j];
    }
  }
  return 0;
}

/* Attention forward, the product whose second matrix multiply (P times V) takes V as a
 * non-K-contiguous operand: V is stored [key][head dim], its reduction index (the key) is
 * the strided one (Triton PR 5223, "Introduction": the second dot operation of flash
 * attention). Written from the definition of scaled softmax attention, per batch-head
 * slice h and query row i:
 *   1. s(j) = scale * sum_d q(i, d) * k(j, d)       for every key j (fp64 dot products);
 *   2. p(j) = exp(s(j) - max_j s(j))                (the shift cancels in step 3 and keeps
 *                                                    every exponent <= 0);
 *   3. o(i, d) = sum_j p(j) * v(j, d) / sum_j p(j)  (fp64 sums, one division).
 * q is [BH][Sq][D], k and v are [BH][Sk][D], o is [BH][Sq][D], all row-major with the head
 * dimension contiguous. Rows r = h * Sq + i in [row_begin, row_end) are computed; o holds
 * them consecutively. exp is the C library's. */
int oracle_attention_f64(const double* q, const double* k, const double* v, int64_t BH,
                         int64_t Sq, int64_t Sk, int64_t D, double scale, int64_t row_begin,
                         int64_t row_end, double* o) {
  if (row_begin < 0 || row_end > BH * Sq || row_begin > row_end || Sk < 1 || D < 1) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = row_begin; r < row_end; ++r) {
    const int64_t h = r / Sq;
    const double* qi = q + r * D;
    const double* kh = k + h * Sk * D;
    const double* vh = v + h * Sk * D;
    double* oi = o + (r - row_begin) * D;
    double* sj = (double*)malloc((size_t)Sk * sizeof(double));
    double smax = -INFINITY;
    for (int64_t j = 0; j < Sk; ++j) {
      double acc = 0.0;
      for (int64_t d = 0; d < D; ++d) acc += qi[d] * kh[j * D + d];
      sj[j] = scale * acc;
      if (sj[j] > smax) smax = sj[j];
    }
    double denom = 0.0;
    for (int64_t d = 0; d < D; ++d) oi[d] = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
      const double pj = exp(sj[j] - smax);
      denom += pj;
      for (int64_t d = 0; d < D; ++d) oi[d] += pj * vh[j * D + d];
    }
    for (int64_t d = 0; d < D; ++d) oi[d] /= denom;
    free(sj);
  }
  return 0;
}

/* Number of threads the OpenMP loop above runs with. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
