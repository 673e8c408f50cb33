/*
 * attn_bwd_ex_oracle.c -- the oracle for the attention backward pass on
 * general shapes (Nq queries against Nk keys, bottom-right causal mask).
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load this code.
 * It shares no source, header, table or helper with the HIP library.
 *
 * The same plain derivative as attn_bwd_oracle.c (dV = P^T dO, dP = dO V^T,
 * delta = rowsum(dO o O), dS = P o (dP - delta), dQ = scale dS K,
 * dK = scale dS^T Q), written with rectangular Nq x Nk matrices, one head at
 * a time, in fp64.  Build with plain -O2, never -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

static double ex_widen_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * General shapes: Nq queries against Nk keys per head, the causal mask
 * aligned bottom-right as in the general-shape forward (key j visible to
 * query i iff j <= i + Nk - Nq).  A query row that sees no key has P = 0,
 * O = 0 and lse = -infinity; it contributes nothing to dK or dV and its dQ
 * row is 0.  Same steps as above with rectangular Nq x Nk matrices.
 */
static int64_t ex_visible(int64_t i, int64_t Nq, int64_t Nk, int causal)
{
    if (!causal) return Nk;
    const int64_t last = i + (Nk - Nq);
    return last < 0 ? 0 : (last + 1 < Nk ? last + 1 : Nk);
}

/* Forward of one head, fp64: o [Nq,d], lse [Nq], p [Nq,Nk] (0 where masked). */
int attn_fwd_oracle_head_ex_f64(const double *q, const double *k, const double *v,
                                int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                                double *o, double *lse, double *p)
{
    if (!q || !o || !lse || !p || Nq <= 0 || Nk < 0 || d <= 0) return ORACLE_ERR_ARG;
    if (Nk > 0 && (!k || !v)) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < Nq; ++i) {
        const int64_t nvis = ex_visible(i, Nq, Nk, causal);
        double *pi = p + i * Nk;
        for (int64_t j = 0; j < Nk; ++j) pi[j] = 0.0;
        for (int64_t t = 0; t < d; ++t) o[i * d + t] = 0.0;
        if (nvis == 0) { lse[i] = -INFINITY; continue; }
        double m = -INFINITY;
        for (int64_t j = 0; j < nvis; ++j) {
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
 * Backward of one head, fp64: dq [Nq,d], dk and dv [Nk,d], delta [Nq]; o and
 * lse receive the forward values used.  `scratch` holds 2*Nq*Nk doubles.
 */
int attn_bwd_oracle_head_ex_f64(const double *q, const double *k, const double *v,
                                const double *dout, int64_t Nq, int64_t Nk, int64_t d,
                                int causal, double scale, double *dq, double *dk, double *dv,
                                double *delta, double *o, double *lse, double *scratch)
{
    if (!dout || !dq || !delta || !scratch || (Nk > 0 && (!dk || !dv))) return ORACLE_ERR_ARG;
    double *p = scratch;             /* P,  Nq x Nk */
    double *ds = scratch + Nq * Nk;  /* dS, Nq x Nk */
    int st = attn_fwd_oracle_head_ex_f64(q, k, v, Nq, Nk, d, causal, scale, o, lse, p);
    if (st != ORACLE_OK) return st;
    for (int64_t i = 0; i < Nq; ++i) {
        double acc = 0.0;
        for (int64_t t = 0; t < d; ++t) acc += dout[i * d + t] * o[i * d + t];
        delta[i] = acc;
    }
    for (int64_t i = 0; i < Nq; ++i) {
        const int64_t nvis = ex_visible(i, Nq, Nk, causal);
        for (int64_t j = 0; j < Nk; ++j) {
            if (j >= nvis) { ds[i * Nk + j] = 0.0; continue; }  /* masked */
            double dp = 0.0;
            for (int64_t t = 0; t < d; ++t) dp += dout[i * d + t] * v[j * d + t];
            ds[i * Nk + j] = p[i * Nk + j] * (dp - delta[i]);
        }
    }
    for (int64_t j = 0; j < Nk; ++j)
        for (int64_t t = 0; t < d; ++t) {
            double av = 0.0, ak = 0.0;
            for (int64_t i = 0; i < Nq; ++i) {
                av += p[i * Nk + j] * dout[i * d + t];
                ak += ds[i * Nk + j] * q[i * d + t];
            }
            dv[j * d + t] = av;
            dk[j * d + t] = scale * ak;
        }
    for (int64_t i = 0; i < Nq; ++i)
        for (int64_t t = 0; t < d; ++t) {
            double aq = 0.0;
            for (int64_t j = 0; j < Nk; ++j) aq += ds[i * Nk + j] * k[j * d + t];
            dq[i * d + t] = scale * aq;
        }
    return ORACLE_OK;
}

/*
 * Heads [h_begin, h_end) of bf16 inputs q, dout [B*H, Nq, d] and k, v
 * [B*H, Nk, d].  Outputs fp64: dq [B*H, Nq, d], dk and dv [B*H, Nk, d],
 * delta [B*H, Nq].
 */
int attn_bwd_oracle_heads_ex(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const uint16_t *dout, int64_t BH, int64_t Nq, int64_t Nk, int64_t d,
                             int causal, double scale, int64_t h_begin, int64_t h_end,
                             double *dq, double *dk, double *dv, double *delta)
{
    if (!q || !dout || !dq || !delta || (Nk > 0 && (!k || !v || !dk || !dv))) return ORACLE_ERR_ARG;
    if (BH <= 0 || Nq <= 0 || Nk < 0 || d <= 0 || h_begin < 0 || h_end > BH || h_begin > h_end)
        return ORACLE_ERR_ARG;
    const int64_t nqd = Nq * d, nkd = Nk * d;
    double *buf = (double *)malloc((size_t)(3 * nqd + 2 * nkd + Nq + 2 * Nq * Nk + 1) * sizeof(double));
    if (!buf) return ORACLE_ERR_NOMEM;
    double *qf = buf, *gf = qf + nqd, *of = gf + nqd, *kf = of + nqd, *vf = kf + nkd;
    double *lse = vf + nkd, *scratch = lse + Nq;
    int st = ORACLE_OK;
    for (int64_t hh = h_begin; hh < h_end && st == ORACLE_OK; ++hh) {
        for (int64_t x = 0; x < nqd; ++x) {
            qf[x] = ex_widen_bf16(q[hh * nqd + x]);
            gf[x] = ex_widen_bf16(dout[hh * nqd + x]);
        }
        for (int64_t x = 0; x < nkd; ++x) {
            kf[x] = ex_widen_bf16(k[hh * nkd + x]);
            vf[x] = ex_widen_bf16(v[hh * nkd + x]);
        }
        st = attn_bwd_oracle_head_ex_f64(qf, kf, vf, gf, Nq, Nk, d, causal, scale, dq + hh * nqd,
                                         dk + hh * nkd, dv + hh * nkd, delta + hh * Nq, of, lse,
                                         scratch);
    }
    free(buf);
    return st;
}
