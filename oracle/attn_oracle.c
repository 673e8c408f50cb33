/*
 * attn_oracle.c -- the oracle for the fused attention forward pass.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load this code.
 * It shares no source, header, table or helper with the HIP library.
 *
 * What it computes (plain definition, fp64, one query row at a time):
 *
 *   For a head (b, h) and query row i, with the visible key set
 *   A(i) = {0 .. N-1} (non-causal) or {0 .. i} (causal, diagonal included):
 *
 *     s_j  = scale * sum_t q[i,t] * k[j,t]              j in A(i)
 *     m    = max_j s_j
 *     l    = sum_j exp(s_j - m)
 *     o[t] = ( sum_j exp(s_j - m) * v[j,t] ) / l
 *     lse  = m + ln(l)                                  (= ln sum_j exp(s_j))
 *
 * Sources on the pages:
 *   - ThunderKittens write-up (88811315.cn), "RTX 4090 flash-attention
 *     example" and "H100 FlashAttention-2 forward example": the per-block
 *     running-max / running-normaliser recurrence.  Its fixed point, after the
 *     last key block, is exactly the softmax-weighted sum above; the oracle
 *     evaluates that fixed point directly (two passes, no running max, no
 *     blocking), so it shares no algorithmic structure with a streaming kernel.
 *   - Same examples: the temperature 1/sqrt(d) multiplies the scores.  Here the
 *     scale is applied exactly in fp64 to the score (the examples round the
 *     scaled Q to bf16; that extra rounding is deliberately not reproduced).
 *   - The log-sum-exp output and the causal mask are not in the printed
 *     examples.  Readings taken: lse is the natural log of the sum of exp of the
 *     scaled scores; causal means key j is visible to query i iff j <= i.
 *
 * Inputs are bf16 bit patterns (uint16), [B,H,N,d] contiguous row-major.  Each
 * bf16 value is widened exactly to double.  Accumulation, exp and log are fp64
 * (libm exp/log).  Build with plain -O2, never -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

/* Exact widening of a bf16 bit pattern: bf16 is the top half of an fp32. */
static double widen_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * One query row.  `scores` is caller scratch of at least N doubles.
 * Writes d doubles to o_row and one double to *lse_out.
 */
int attn_oracle_row(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    int64_t B, int64_t H, int64_t N, int64_t d,
                    int causal, double scale,
                    int64_t b, int64_t h, int64_t i,
                    double *o_row, double *lse_out, double *scores)
{
    if (!q || !k || !v || !o_row || !lse_out || !scores) return ORACLE_ERR_ARG;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return ORACLE_ERR_ARG;
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N) return ORACLE_ERR_ARG;

    const int64_t head = (b * H + h) * N * d;
    const uint16_t *qi = q + head + i * d;
    const uint16_t *kh = k + head;
    const uint16_t *vh = v + head;
    const int64_t nvis = causal ? i + 1 : N;

    /* Pass 1: every visible scaled score, and their maximum. */
    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) {
        double dot = 0.0;
        for (int64_t t = 0; t < d; ++t)
            dot += widen_bf16(qi[t]) * widen_bf16(kh[j * d + t]);
        scores[j] = scale * dot;
        if (scores[j] > m) m = scores[j];
    }

    /* Pass 2: softmax weights, their sum, and the weighted sum of values. */
    for (int64_t t = 0; t < d; ++t) o_row[t] = 0.0;
    double l = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const double w = exp(scores[j] - m);
        l += w;
        for (int64_t t = 0; t < d; ++t)
            o_row[t] += w * widen_bf16(vh[j * d + t]);
    }
    for (int64_t t = 0; t < d; ++t) o_row[t] /= l;
    *lse_out = m + log(l);
    return ORACLE_OK;
}

/*
 * A list of rows, each named by its flat index r = (b*H + h)*N + i.
 * o_out is [nrows, d], lse_out is [nrows].  Single-threaded; callers that
 * want several cores split the row list between threads.
 */
int attn_oracle_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int64_t B, int64_t H, int64_t N, int64_t d,
                     int causal, double scale,
                     const int64_t *rows, int64_t nrows,
                     double *o_out, double *lse_out)
{
    if (!rows || !o_out || !lse_out || nrows < 0) return ORACLE_ERR_ARG;
    if (N <= 0) return ORACLE_ERR_ARG;
    double *scores = (double *)malloc((size_t)N * sizeof(double));
    if (!scores) return ORACLE_ERR_NOMEM;
    int status = ORACLE_OK;
    for (int64_t n = 0; n < nrows && status == ORACLE_OK; ++n) {
        const int64_t r = rows[n];
        if (r < 0 || r >= B * H * N) { status = ORACLE_ERR_ARG; break; }
        const int64_t i = r % N;
        const int64_t bh = r / N;
        status = attn_oracle_row(q, k, v, B, H, N, d, causal, scale,
                                 bh / H, bh % H, i,
                                 o_out + n * d, lse_out + n, scores);
    }
    free(scores);
    return status;
}

/*
 * General shapes: Nq queries against Nk keys per head.  q and o are
 * [B,H,Nq,d], k and v are [B,H,Nk,d].  Causal masks are aligned bottom-right
 * (the convention for a block of queries that ends where the keys end): key
 * j is visible to query i iff j <= i + (Nk - Nq); with Nq = Nk this is the
 * mask of attn_oracle_row.  A row that sees no key (possible when Nq > Nk)
 * has no softmax; it is defined here as o = 0 and lse = -infinity, the
 * values that make it vanish from a log-sum-exp merge of partial results.
 * `scores` is caller scratch of at least Nk doubles.
 */
int attn_oracle_row_ex(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                       int causal, double scale,
                       int64_t b, int64_t h, int64_t i,
                       double *o_row, double *lse_out, double *scores)
{
    if (!q || !k || !v || !o_row || !lse_out || !scores) return ORACLE_ERR_ARG;
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return ORACLE_ERR_ARG;
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Nq) return ORACLE_ERR_ARG;

    const uint16_t *qi = q + ((b * H + h) * Nq + i) * d;
    const uint16_t *kh = k + (b * H + h) * Nk * d;
    const uint16_t *vh = v + (b * H + h) * Nk * d;
    int64_t nvis = Nk;
    if (causal) {
        const int64_t last = i + (Nk - Nq);      /* last visible key */
        nvis = last < 0 ? 0 : (last + 1 < Nk ? last + 1 : Nk);
    }
    for (int64_t t = 0; t < d; ++t) o_row[t] = 0.0;
    if (nvis == 0) {
        *lse_out = -INFINITY;
        return ORACLE_OK;
    }

    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) {
        double dot = 0.0;
        for (int64_t t = 0; t < d; ++t)
            dot += widen_bf16(qi[t]) * widen_bf16(kh[j * d + t]);
        scores[j] = scale * dot;
        if (scores[j] > m) m = scores[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const double w = exp(scores[j] - m);
        l += w;
        for (int64_t t = 0; t < d; ++t)
            o_row[t] += w * widen_bf16(vh[j * d + t]);
    }
    for (int64_t t = 0; t < d; ++t) o_row[t] /= l;
    *lse_out = m + log(l);
    return ORACLE_OK;
}

/* Rows r = (b*H + h)*Nq + i of the general-shape problem; see above. */
int attn_oracle_rows_ex(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                        int causal, double scale,
                        const int64_t *rows, int64_t nrows,
                        double *o_out, double *lse_out)
{
    if (!rows || !o_out || !lse_out || nrows < 0 || Nk <= 0 || Nq <= 0) return ORACLE_ERR_ARG;
    double *scores = (double *)malloc((size_t)Nk * sizeof(double));
    if (!scores) return ORACLE_ERR_NOMEM;
    int status = ORACLE_OK;
    for (int64_t n = 0; n < nrows && status == ORACLE_OK; ++n) {
        const int64_t r = rows[n];
        if (r < 0 || r >= B * H * Nq) { status = ORACLE_ERR_ARG; break; }
        const int64_t bh = r / Nq;
        status = attn_oracle_row_ex(q, k, v, B, H, Nq, Nk, d, causal, scale,
                                    bh / H, bh % H, r % Nq,
                                    o_out + n * d, lse_out + n, scores);
    }
    free(scores);
    return status;
}
