/*
 * attn_bwd.h -- C ABI of the MI355X (gfx950) attention backward pass.
 *
 * The pages benchmark the flash-attention backward pass next to the forward
 * (ThunderKittens write-ups: the forward examples, and the write-up's
 * statements about its backward kernels) but print no listing of it.  What
 * this library computes is the derivative of the forward of attn_fwd.h,
 * O = softmax(scale * Q K^T) V (causal: key j visible to query i iff j <= i),
 * for a scalar loss whose gradient with respect to O is dO:
 *
 *   P       = softmax(scale * Q K^T)        (recomputed from Q, K and the
 *                                            forward's LSE: P = exp(S - lse))
 *   delta_i = sum_t dO[i,t] * O[i,t]
 *   dV      = P^T dO
 *   dS      = P o (dO V^T - delta)          (o: elementwise, delta per row)
 *   dQ      = scale * dS K
 *   dK      = scale * dS^T Q
 *
 * Inputs are bf16, products accumulate in fp32, P and dS are rounded to bf16
 * as MFMA operands, dQ/dK/dV are rounded to bf16 (round-to-nearest-even).
 * Status codes are those of attn_fwd.h.  No HIP header is needed by callers.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include "attn_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_bwd -- enqueue the attention backward on `stream`.
 *
 *   q, k, v  device pointers, bf16 [B, H, N, d] contiguous (d fastest), the
 *            forward's inputs.  Read only.
 *   o        bf16 [B, H, N, d]: the forward's output.  Read only.
 *   lse      fp32 [B, H, N]: the forward's log-sum-exp (natural log), as
 *            written by attn_fwd with the same q, k, causal and scale.
 *   dout     bf16 [B, H, N, d]: gradient of the loss with respect to o.
 *   dq, dk, dv  bf16 [B, H, N, d]: written completely.
 *   delta    fp32 [B, H, N]: written completely with rowsum(dout * o); it is
 *            also the library's only intermediate (read back by the later
 *            kernels of the same call), so it must not alias any other
 *            argument.
 *   B, H, N, d, causal, scale: as for attn_fwd (d = 32, 64, 96, 128 or 256, any N >= 0).
 *   stream   a hipStream_t cast to void*; NULL means the default stream.
 *
 * All pointers are 16-byte aligned device pointers; outputs must not overlap
 * inputs.  The library allocates nothing; calls are asynchronous, re-entrant
 * and may run concurrently on different streams.  Every argument check runs
 * before any HIP call; on an error return nothing has been launched.
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *o,
             const float *lse, const void *dout,
             void *dq, void *dk, void *dv, float *delta,
             int B, int H, int N, int d,
             int causal, float scale,
             void *stream);

/*
 * attn_bwd_ex -- the same backward for Nq queries against Nk keys per head,
 * the derivative of attn_fwd_ex (attn_fwd.h): causal masks are aligned
 * bottom-right (key j visible to query i iff j <= i + Nk - Nq).
 *
 *   q, o, dout, dq   [B, H, Nq, d];   k, v, dk, dv   [B, H, Nk, d];
 *   lse, delta       [B, H, Nq]       (lse from attn_fwd_ex on the same
 *                                      problem; -inf for rows that see no key)
 *
 * A query row that sees no key gets dq = 0 and delta = 0 and adds nothing to
 * dk or dv; with Nq = 0, dk = dv = 0.  Query-side pointers (q, o, lse, dout,
 * dq, delta) may be NULL when Nq = 0 and key-side ones (k, v, dk, dv) when
 * Nk = 0.  Every other argument, and ownership, errors and semantics, are as
 * for attn_bwd; with Nq = Nk the call is exactly attn_bwd.
 */
int attn_bwd_ex(const void *q, const void *k, const void *v, const void *o,
                const float *lse, const void *dout,
                void *dq, void *dk, void *dv, float *delta,
                int B, int H, int Nq, int Nk, int d,
                int causal, float scale,
                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
