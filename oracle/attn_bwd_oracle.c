/*
 * attn_bwd_oracle.c -- the oracle for the attention backward pass.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load this code.
 * It shares no source, header, table or helper with the HIP library.
 *
 * The pages name the backward pass (the flash-attention backward that the
 * ThunderKittens write-ups benchmark) but print no listing of it, so this file
 * is the plain derivative of the forward definition, written out with full
 * N x N matrices, one head at a time, in fp64:
 *
 *   S  = scale * Q K^T                          (visible entries only)
 *   P  = row-wise softmax of S                  (masked entries are 0)
 *   O  = P V,   lse_i = ln sum_j exp(S_ij)
 *   given dO (the gradient of a scalar loss with respect to O):
 *   dV    = P^T dO
 *   dP    = dO V^T
 *   delta_i = sum_t dO[i,t] * O[i,t]            (= sum_j P_ij dP_ij)
 *   dS    = P o (dP - delta 1^T)                (o: elementwise)
 *   dQ    = scale * dS K
 *   dK    = scale * dS^T Q
 *
 * The softmax Jacobian gives dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik); the
 * inner sum equals delta_i because O_i = sum_k P_ik V_k.  Visible keys: all j
 * (non-causal) or j <= i (causal, the forward's convention).
 *
 * Two entry points: one on fp64 inputs (used by the finite-difference pins),
 * one on bf16 bit patterns, widened exactly to fp64.  Build with plain -O2,
 * never -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

static double bwd_widen_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Forward of one head on fp64 inputs: o [N,d], lse [N].  `p` is caller
 * scratch of N*N doubles and receives the probabilities (0 where masked).
 */
int attn_fwd_oracle_head_f64(const double *q, const double *k, const double *v,
                             int64_t N, int64_t d, int causal, double scale,
                             double *o, double *lse, double *p)
{
    if (!q || !k || !v || !o || !lse || !p || N <= 0 || d <= 0) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < N; ++i) {
        const int64_t nvis = causal ? i + 1 : N;
        double *pi = p + i * N;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            if (j >= nvis) { pi[j] = 0.0; continue; }
            double dot = 0.0;
            for (int64_t t = 0; t < d; ++t) dot += q[i * d + t] * k[j * d + t];
            pi[j] = scale * dot;
            if (pi[j] > m) m = pi[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nvis; ++j) {
            pi[j] = exp(pi[j] - m);
            l += pi[j];
        }
        for (int64_t j = 0; j < nvis; ++j) pi[j] /= l;
        lse[i] = m + log(l);
        for (int64_t t = 0; t < d; ++t) {
            double acc = 0.0;
            for (int64_t j = 0; j < nvis; ++j) acc += pi[j] * v[j * d + t];
            o[i * d + t] = acc;
        }
    }
    return ORACLE_OK;
}

/*
 * Backward of one head on fp64 inputs.  Outputs dq, dk, dv [N,d] and delta
 * [N]; o [N,d] and lse [N] receive the forward values used.  `scratch` holds
 * at least 2*N*N doubles.
 */
int attn_bwd_oracle_head_f64(const double *q, const double *k, const double *v,
                             const double *dout, int64_t N, int64_t d, int causal,
                             double scale, double *dq, double *dk, double *dv,
                             double *delta, double *o, double *lse, double *scratch)
{
    if (!dout || !dq || !dk || !dv || !delta || !scratch) return ORACLE_ERR_ARG;
    double *p = scratch;           /* P,  N x N */
    double *ds = scratch + N * N;  /* dS, N x N */
    int st = attn_fwd_oracle_head_f64(q, k, v, N, d, causal, scale, o, lse, p);
    if (st != ORACLE_OK) return st;

    /* delta_i = dO_i . O_i */
    for (int64_t i = 0; i < N; ++i) {
        double acc = 0.0;
        for (int64_t t = 0; t < d; ++t) acc += dout[i * d + t] * o[i * d + t];
        delta[i] = acc;
    }
    /* dP_ij = dO_i . V_j, then dS = P o (dP - delta) */
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < N; ++j) {
            if (causal && j > i) { ds[i * N + j] = 0.0; continue; }  /* masked */
            const double pij = p[i * N + j];
            double dp = 0.0;
            for (int64_t t = 0; t < d; ++t) dp += dout[i * d + t] * v[j * d + t];
            ds[i * N + j] = pij * (dp - delta[i]);
        }
    /* dV = P^T dO,  dK = scale * dS^T Q */
    for (int64_t j = 0; j < N; ++j)
        for (int64_t t = 0; t < d; ++t) {
            double av = 0.0, ak = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                av += p[i * N + j] * dout[i * d + t];
                ak += ds[i * N + j] * q[i * d + t];
            }
            dv[j * d + t] = av;
            dk[j * d + t] = scale * ak;
        }
    /* dQ = scale * dS K */
    for (int64_t i = 0; i < N; ++i)
        for (int64_t t = 0; t < d; ++t) {
            double aq = 0.0;
            for (int64_t j = 0; j < N; ++j) aq += ds[i * N + j] * k[j * d + t];
            dq[i * d + t] = scale * aq;
        }
    return ORACLE_OK;
}

/*
 * Backward of heads [h_begin, h_end) of [B,H,N,d] bf16 inputs (flat head index
 * b*H + h).  Outputs are fp64 arrays laid out [B*H, N, d] (dq, dk, dv) and
 * [B*H, N] (delta), written only for the listed heads.  Single-threaded;
 * callers split heads between threads.
 */
int attn_bwd_oracle_heads(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const uint16_t *dout, int64_t BH, int64_t N, int64_t d,
                          int causal, double scale, int64_t h_begin, int64_t h_end,
                          double *dq, double *dk, double *dv, double *delta)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !delta) return ORACLE_ERR_ARG;
    if (BH <= 0 || N <= 0 || d <= 0 || h_begin < 0 || h_end > BH || h_begin > h_end)
        return ORACLE_ERR_ARG;
    const int64_t nd = N * d;
    double *buf = (double *)malloc((size_t)(4 * nd + nd + N + 2 * N * N) * sizeof(double));
    if (!buf) return ORACLE_ERR_NOMEM;
    double *qf = buf, *kf = qf + nd, *vf = kf + nd, *gf = vf + nd, *of = gf + nd;
    double *lse = of + nd, *scratch = lse + N;
    int st = ORACLE_OK;
    for (int64_t hh = h_begin; hh < h_end && st == ORACLE_OK; ++hh) {
        const int64_t off = hh * nd;
        for (int64_t x = 0; x < nd; ++x) {
            qf[x] = bwd_widen_bf16(q[off + x]);
            kf[x] = bwd_widen_bf16(k[off + x]);
            vf[x] = bwd_widen_bf16(v[off + x]);
            gf[x] = bwd_widen_bf16(dout[off + x]);
        }
        st = attn_bwd_oracle_head_f64(qf, kf, vf, gf, N, d, causal, scale, dq + off, dk + off,
                                      dv + off, delta + hh * N, of, lse, scratch);
    }
    free(buf);
    return st;
}
