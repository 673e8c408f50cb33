/*
 * gemm_oracle.c -- the oracle for the bf16 matrix product.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load this code.
 * It shares no source, header, table or helper with the HIP library.
 *
 * What it computes (plain definition, fp64):
 *
 *     c[m][n] = sum_{k < K} a[m][k] * b(k, n)
 *
 * with A row-major [M, K] and B either row-major [K, N] (b(k, n) = b[k][n],
 * C = A B) or row-major [N, K] (b(k, n) = b[n][k], C = A B^T, the layout of a
 * weight matrix applied to row vectors).
 *
 * Source on the pages: the ThunderKittens paper summary (abstract and key
 * points) names GEMM, benchmarked against cuBLAS, as one of the framework's
 * kernels; no listing, layout or precision is printed.  Readings taken: bf16
 * inputs and a product accumulated exactly (here fp64, sequential in k), the
 * plain matrix product of linear algebra.
 *
 * Inputs are bf16 bit patterns (uint16), contiguous row-major.  Each value is
 * widened exactly to double.  Build with plain -O2, never -ffast-math.
 */
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1

static double widen_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Rows `rows[0..nrows)` of C, written to c_out [nrows, N] (fp64).
 * b_layout 0: B is [K, N]; 1: B is [N, K].  K may be 0 (C = 0).
 */
int gemm_oracle_rows(const uint16_t *a, const uint16_t *b, int64_t M, int64_t N, int64_t K,
                     int b_layout, const int64_t *rows, int64_t nrows, double *c_out)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0) return ORACLE_ERR_ARG;
    if (b_layout != 0 && b_layout != 1) return ORACLE_ERR_ARG;
    if (nrows > 0 && (!rows || !c_out)) return ORACLE_ERR_ARG;
    if (K > 0 && nrows > 0 && (!a || !b)) return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t m = rows[r];
        if (m < 0 || m >= M) return ORACLE_ERR_ARG;
        const uint16_t *arow = a + m * K;
        double *crow = c_out + r * N;
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const uint16_t bk = b_layout == 0 ? b[k * N + n] : b[n * K + k];
                sum += widen_bf16(arow[k]) * widen_bf16(bk);
            }
            crow[n] = sum;
        }
    }
    return ORACLE_OK;
}
