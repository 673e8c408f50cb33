/*
 * attn_gemm.h -- C ABI of the bf16 matrix product on gfx950 (MI355X) MFMA.
 *
 * The operation (the ThunderKittens paper summary, abstract and key points,
 * lists GEMM beside attention as a kernel measured against the vendor BLAS;
 * no listing is printed, so the plain definition is taken):
 *
 *     C[m][n] = sum_{k < K} A[m][k] * B(k, n)          for m < M, n < N
 *
 * A is row-major [M, K].  B is row-major [K, N] (ATTN_GEMM_NN: C = A B) or
 * row-major [N, K] (ATTN_GEMM_NT: C = A B^T, a weight matrix applied to the
 * rows of A).  Inputs are bf16, products are accumulated in fp32 on the
 * matrix cores, and C is rounded to bf16 (round-to-nearest-even), row-major
 * [M, N].
 *
 * Status codes are those of attn_fwd.h.  No HIP header is needed to call
 * this library.
 */
#ifndef ATTN_GEMM_H
#define ATTN_GEMM_H

#include "attn_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

enum attn_gemm_layout {
    ATTN_GEMM_NN = 0, /* B is [K, N]:  C = A B   */
    ATTN_GEMM_NT = 1  /* B is [N, K]:  C = A B^T */
};

/*
 * attn_gemm_bf16 -- enqueue C = A B (or A B^T) on `stream`.
 *
 *   a        device pointer, bf16 bits, [M, K] row-major, 16-byte aligned.
 *   b        device pointer, bf16 bits, [K, N] (NN) or [N, K] (NT) row-major,
 *            16-byte aligned.
 *   c        device pointer, bf16 [M, N] row-major, 16-byte aligned.  Written
 *            completely (all zeros when K = 0).
 *   M, N, K  sizes, >= 0.  N and K must be multiples of 8 (every row starts
 *            16-byte aligned) and below 2^22 (a 256-row tile's byte offsets
 *            fit an int); M is any int.
 *   layout   ATTN_GEMM_NN or ATTN_GEMM_NT.
 *   stream   a hipStream_t cast to void*; NULL means the default stream.
 *
 * Errors (checked before any HIP call; nothing is written on error):
 *   ATTN_ERR_SHAPE   a size is negative, N or K is not a multiple of 8, a
 *                    size limit above is exceeded, or layout is unknown;
 *   ATTN_ERR_NULL    a pointer is NULL while M*N > 0 (a and b may be NULL
 *                    when K = 0);
 *   ATTN_ERR_ALIGN   a pointer is not 16-byte aligned;
 *   ATTN_ERR_DEVICE  the current device is not a gfx950 GPU;
 *   ATTN_ERR_HIP     the launch failed.
 *
 * Ownership and semantics: as for attn_fwd (caller-owned buffers, nothing
 * allocated, asynchronous; c must not overlap a or b).
 */
int attn_gemm_bf16(const void *a, const void *b, void *c, int M, int N, int K, int layout,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GEMM_H */
