/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * The operation (flash-attention forward; ThunderKittens write-up,
 * 88811315.cn, "RTX 4090 flash-attention example" and "H100 FlashAttention-2
 * forward example"; the same kernels are summarised on GeekNews, "Ejemplo de
 * FlashAttention y rendimiento"):
 *
 *   for every batch b < B, head h < H and query row i < N
 *     s_ij   = scale * sum_t q[b,h,i,t] * k[b,h,j,t]        for visible j
 *     o[b,h,i,:] = sum_j softmax_j(s_i.) * v[b,h,j,:]
 *     lse[b,h,i] = ln sum_j exp(s_ij)                          (natural log)
 *
 * where the visible keys are all j < N, or j <= i when `causal` is non-zero
 * (query i sees keys 0..i, diagonal included).  The N x N score matrix is
 * never stored: keys and values are streamed in tiles and a running row
 * maximum and normaliser are kept per query, the recurrence those examples
 * print.  Inputs are bf16, products are accumulated in fp32, softmax runs in
 * fp32, the probabilities are rounded to bf16 for the second product (as in
 * those examples), O is rounded to bf16 (round-to-nearest-even) and the
 * log-sum-exp is fp32.  The examples multiply Q by the temperature in bf16;
 * this library applies `scale` to the fp32 scores instead.
 *
 * No HIP header is needed to call this library.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every argument check runs before any HIP call; on an error
 * return nothing has been launched and no output byte has been written. */
enum attn_fwd_status {
    ATTN_OK = 0,               /* launched (or nothing to do)                  */
    ATTN_ERR_NULL = 1,         /* a pointer is NULL while B*H*N > 0            */
    ATTN_ERR_SHAPE = 2,        /* B, H or N negative, or the sizes overflow    */
    ATTN_ERR_HEAD_DIM = 3,     /* d not in {32, 64, 96, 128, 256} (forward)   */
    ATTN_ERR_SEQ_MULTIPLE = 4, /* reserved: any N >= 0 is accepted             */
    ATTN_ERR_ALIGN = 5,        /* a pointer is not 16-byte aligned             */
    ATTN_ERR_SCALE = 6,        /* scale is not finite or not > 0               */
    ATTN_ERR_HIP = 7,          /* the HIP runtime reported an error at launch  */
    ATTN_ERR_DEVICE = 8,       /* the current device is not a gfx950 GPU       */
    ATTN_ERR_WORKSPACE = 9     /* attn_fwd_splitkv_noalloc: partial results
                                  larger than its fixed workspace              */
};

/*
 * attn_fwd -- enqueue the fused attention forward on `stream`.
 *
 *   q, k, v  device pointers to bf16 bit patterns, each [B, H, N, d]
 *            contiguous row-major (d fastest), 16-byte aligned.  Read only.
 *   o        device pointer, bf16 [B, H, N, d] contiguous, 16-byte aligned.
 *            Written completely.
 *   lse      device pointer, fp32 [B, H, N] contiguous, 16-byte aligned.
 *            Written completely: natural-log log-sum-exp of each row's
 *            scaled scores.  Required (not optional).
 *   B, H, N  batch, heads, sequence length (queries = keys = N).  Any of them
 *            may be 0 (nothing is launched); N need not be a multiple of any
 *            tile size.  B*H*ceil(N/128) and N*d*2 must fit in an int.
 *   d        head dimension: 32, 64, 96, 128 or 256.  (The examples fix d:
 *            64 on the RTX 4090, 64 or 128 as a template parameter on the
 *            H100; the other sizes are this library's extension, computed
 *            with the same 16-deep MFMA steps and 32-wide output blocks.)
 *   causal   0: every query sees every key.  Non-zero: query i sees keys
 *            0..i (lower-triangular mask, top-left aligned).
 *   scale    multiplies q.k; finite and > 0 (1/sqrt(d) is the usual value).
 *   stream   a hipStream_t cast to void*; NULL means the default stream.
 *
 * Ownership: the caller owns every buffer; the library allocates no device
 * memory and keeps no per-call state.  The only global state is a per-device
 * cache of the device's properties and of the kernels' resident workgroups
 * per CU, each filled once (thread-safely) on the first call that needs it.
 * Calls are re-entrant, may run concurrently on different streams, and may
 * be captured in a HIP graph.
 *
 * Semantics: asynchronous.  ATTN_OK means the kernel was enqueued; results
 * are visible after the stream (or an event on it) is synchronised, and a
 * fault during execution surfaces there, as with any HIP launch.  `o` and
 * `lse` must not overlap q, k or v (not checked).  Non-finite input values
 * give undefined (non-finite) outputs for the rows that see them.
 */
int attn_fwd(const void *q, const void *k, const void *v,
             void *o, float *lse,
             int B, int H, int N, int d,
             int causal, float scale,
             void *stream);

/*
 * attn_fwd_ex -- the same forward for Nq queries against Nk keys per head.
 *
 *   q, o     [B, H, Nq, d];  k, v  [B, H, Nk, d];  lse  [B, H, Nq].
 *   causal   non-zero: the mask is aligned bottom-right, key j is visible to
 *            query i iff j <= i + (Nk - Nq) (the last query sees every key;
 *            with Nq = Nk this is attn_fwd's mask).  A row that sees no key
 *            (Nq > Nk, causal; or Nk = 0) is written as o = 0, lse = -inf, so
 *            that it drops out of a log-sum-exp merge of partial results.
 *
 * Every other argument, and ownership, errors and semantics, are as for
 * attn_fwd (k and v may be NULL when Nk = 0: they are not read).  With
 * Nq = Nk the call is exactly attn_fwd.
 */
int attn_fwd_ex(const void *q, const void *k, const void *v,
                void *o, float *lse,
                int B, int H, int Nq, int Nk, int d,
                int causal, float scale,
                void *stream);

/*
 * attn_fwd_splitkv -- attn_fwd_ex computed as n_splits independent key
 * ranges of whole 64-key tiles, processed by separate workgroups, then merged
 * per row: lse = ln sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s (the
 * result is attn_fwd_ex's up to rounding).  It fills the GPU when
 * B*H*ceil(Nq/256) workgroups are too few, e.g. Nq = 1 against a long Nk.
 *
 *   n_splits  requested number of key ranges, >= 1.  Ranges are
 *             ceil(Nk / n_splits) keys rounded up to a multiple of 64, so the
 *             number used, n_used = ceil(Nk / range), may be smaller;
 *             n_used <= 1 runs attn_fwd_ex directly.
 *   o_part    caller workspace, fp32 [n_splits, B, H, Nq, d] (device, 16-byte
 *             aligned); lse_part  fp32 [n_splits, B, H, Nq].  Only the first
 *             n_used slices are written and read; their contents afterwards
 *             are unspecified.  Either may be NULL when n_used <= 1.
 *
 * Every other argument, and ownership, errors and semantics, are as for
 * attn_fwd_ex.  Two kernels run on `stream` (the splits, then the merge).
 */
int attn_fwd_splitkv(const void *q, const void *k, const void *v,
                     void *o, float *lse,
                     int B, int H, int Nq, int Nk, int d,
                     int causal, float scale,
                     int n_splits, float *o_part, float *lse_part,
                     void *stream);

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv without the workspace
 * arguments, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The partial results live in a fixed 32 MiB array of device memory inside
 * the library (one per GPU, held until the process ends): fp32 partial O
 * [n_used, B, H, Nq, d], then, from the next 256-byte boundary, the partial
 * LSE [n_used, B, H, Nq], with n_used as for attn_fwd_splitkv.  A problem
 * whose partial results do not fit returns ATTN_ERR_WORKSPACE before any HIP
 * call.  The call allocates nothing: the first call on a device looks up the
 * array's device address once.  Every call on one GPU shares that array, so
 * calls that overlap in time on one GPU (different streams or host threads
 * without ordering between them) race and give undefined results; calls
 * ordered on one stream are safe.  Every partial result is written before it
 * is read in the same call, so nothing needs clearing between calls.
 *
 * Every other argument, and the result, errors and semantics, are as for
 * attn_fwd_splitkv (results are identical to it for the same n_splits).
 */
int attn_fwd_splitkv_noalloc(const void *q, const void *k, const void *v,
                             void *o, float *lse,
                             int B, int H, int Nq, int Nk, int d,
                             int causal, float scale, int n_splits,
                             void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *attn_fwd_strerror(int status);

/* ABI version of this header's entry points (currently 4: attn_fwd_ex and
 * attn_fwd_splitkv added to version 1 in 3, attn_fwd_splitkv_noalloc and
 * ATTN_ERR_WORKSPACE in 4). */
int attn_fwd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
