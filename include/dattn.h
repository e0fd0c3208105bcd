/*
 * dattn.h -- C ABI of the attention forward in libdgemm.so (MI355X, gfx950).
 *
 * O = softmax(scale * Q K^T) V for every batch-head slice: the computation whose second
 * product (P times V) is the other non-K-contiguous operand case of the inThreadTranspose
 * page (Triton PR 5223, "Introduction": the second dot operation of flash attention). V is
 * stored [key][head dim], so the reduction index of P * V (the key) is its strided index;
 * the kernel reads it with the same loader as a transposed GEMM operand (128-bit loads of
 * four key rows per thread, a byte-permute transpose in registers, key-contiguous LDS
 * rows with the row permutation of rocm-libraries PR 2487).
 *
 * Conventions are those of dgemm.h: 0 (GEMM_OK) or a negative GEMM_ERR_* status, checks
 * before any GPU work, no printing (unless DGEMM_DEBUG is set), no device synchronisation
 * and no device allocation.
 */
#ifndef DATTN_H
#define DATTN_H

#include <stdint.h>

#include "dgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue the attention forward on `stream` (a hipStream_t; NULL is the default stream).
 *
 * Q: BH x Sq x D, K and V: BH x Sk x D, O: BH x Sq x D; each a packed row-major device
 *   array with the head dimension contiguous (slice h, row i, element d at
 *   (h * rows + i) * D + d), 16-byte aligned. O must not overlap Q, K or V.
 * dtype: GEMM_F16 or GEMM_BF16, for Q, K, V and O alike.
 * scale: the factor applied to Q K^T before the softmax (finite; typically 1/sqrt(D)).
 * Every row of O is sum_j p_j v_j / sum_j p_j with p_j = exp(scale * q.k_j - max), computed
 *   with fp32 scores, fp32 sums and P rounded once to dtype for the second product; O is
 *   rounded once (round to nearest even) to dtype.
 * Supported: D == 128; BH, Sq, Sk >= 1; BH * max(Sq, Sk) * D * 2 below 2^31 bytes
 *   (GEMM_ERR_UNSUPPORTED otherwise). Null pointers, non-positive sizes, an unknown dtype
 *   or a non-finite scale give GEMM_ERR_INVALID_ARG; misaligned pointers
 *   GEMM_ERR_MISALIGNED; no current HIP device GEMM_ERR_NO_DEVICE; a failed launch
 *   GEMM_ERR_HIP. */
int attn_fwd(const void* Q, const void* K, const void* V, void* O, int64_t BH, int64_t Sq,
             int64_t Sk, int64_t D, int dtype, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DATTN_H */
