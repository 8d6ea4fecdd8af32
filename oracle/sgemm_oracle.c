/*
 * Plain CPU oracle for C = alpha * op(A) * op(B) + beta * C   (TEST INFRASTRUCTURE)
 *
 * This file is test infrastructure. Only the tests, the smoke check and the
 * bench's CPU-baseline leg may load it. The GPU library never links,
 * includes or calls it, and it shares no code, header or helper with that
 * library.
 *
 * What it computes is the textbook definition of GEMM: "Optimising fp32 GEMM
 * on A100", section "What is GEMM?" (C = alpha*(A x B) + beta*C, A is M x K,
 * B is K x N, and the plain triple loop that sums over k with C starting at
 * zero). "How to get a matmul kernel into the top percentile (worklog)",
 * section "Starting Point", gives the same element-wise sum.
 *
 * Precision: every product of two binary32 values is exact in binary64
 * (24 + 24 significand bits <= 53), so the only rounding is the binary64
 * summation, done in ascending k for every element. The same loop also sums
 * |a_ik * b_kj|, which the acceptance bound needs.
 *
 * Storage is row-major with explicit leading dimensions:
 *   op(A)(i,k) = A[i*lda + k]  if transA == 0,  A[k*lda + i]  if transA == 1
 *   op(B)(k,j) = B[k*ldb + j]  if transB == 0,  B[j*ldb + k]  if transB == 1
 *   Cin(i,j)   = Cin[i*ldc + j]
 * When beta == 0 the input C is not read, and when alpha == 0 neither A nor B
 * is read (the BLAS convention; the pages only ever use alpha = 1, beta = 0):
 * the result is then alpha * sum, respectively beta * C, whatever the
 * unread operand held (NaN included).
 *
 * Outputs are dense binary64 arrays with row length N.
 *
 * Parallelism: rows (or requested elements) are independent, so an OpenMP
 * loop over them changes nothing in the arithmetic of any one element.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

static double op_a(const float* A, int64_t lda, int transA, int64_t i, int64_t k)
{
    return transA ? (double)A[k * lda + i] : (double)A[i * lda + k];
}

static double op_b(const float* B, int64_t ldb, int transB, int64_t k, int64_t j)
{
    return transB ? (double)B[j * ldb + k] : (double)B[k * ldb + j];
}

/* One output element, straight from the definition. */
static void one_element(int transA, int transB, int64_t K, double alpha,
                        const float* A, int64_t lda, const float* B, int64_t ldb,
                        double beta, const float* Cin, int64_t ldc,
                        int64_t i, int64_t j, double* cref, double* sabs)
{
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; alpha != 0.0 && k < K; ++k) {
        double p = op_a(A, lda, transA, i, k) * op_b(B, ldb, transB, k, j);
        s += p;
        sa += fabs(p);
    }
    double c = alpha * s;
    if (beta != 0.0)
        c += beta * (double)Cin[i * ldc + j];
    *cref = c;
    *sabs = sa;
}

/*
 * Selected elements (ii[t], jj[t]) for t in [0, n). Used at sizes where the
 * whole product is too slow on the host.
 */
int oracle_gemm_elems(int transA, int transB, int64_t M, int64_t N, int64_t K,
                      double alpha, const float* A, int64_t lda,
                      const float* B, int64_t ldb, double beta,
                      const float* Cin, int64_t ldc,
                      const int64_t* ii, const int64_t* jj, int64_t n,
                      double* cref, double* sabs)
{
    if (M < 0 || N < 0 || K < 0 || n < 0)
        return 1;
    for (int64_t t = 0; t < n; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
            return 2;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < n; ++t)
        one_element(transA, transB, K, alpha, A, lda, B, ldb, beta, Cin, ldc,
                    ii[t], jj[t], &cref[t], &sabs[t]);
    return 0;
}

/*
 * Whole rows. rows == NULL means rows 0..M-1 (then nrows must equal M).
 * Output t*N + j holds element (rows[t], j).
 *
 * Per row the loop order is k outer, j inner, with one binary64 accumulator
 * per j; each element still sees its terms in ascending k, so the result is
 * the same number one_element() gives. op(B) with transB == 1 is first copied
 * into a K x N array (a plain transpose, no arithmetic) so the inner loop
 * walks memory in order.
 */
int oracle_gemm_rows(int transA, int transB, int64_t M, int64_t N, int64_t K,
                     double alpha, const float* A, int64_t lda,
                     const float* B, int64_t ldb, double beta,
                     const float* Cin, int64_t ldc,
                     const int64_t* rows, int64_t nrows,
                     double* cref, double* sabs)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0)
        return 1;
    if (!rows && nrows != M)
        return 2;
    if (rows)
        for (int64_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= M)
                return 2;

    const float* bk = B;   /* op(B) as K x N, row length bld */
    int64_t bld = ldb;
    float* bt = NULL;
    if (transB && alpha != 0.0 && K > 0 && N > 0) {
        bt = (float*)malloc((size_t)K * (size_t)N * sizeof(float));
        if (!bt)
            return 3;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t j = 0; j < N; ++j)
                bt[k * N + j] = B[j * ldb + k];
        bk = bt;
        bld = N;
    }

    int status = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double* sa = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!s || !sa) {
#pragma omp atomic write
            status = 3;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < nrows; ++t) {
                int64_t i = rows ? rows[t] : t;
                for (int64_t j = 0; j < N; ++j) {
                    s[j] = 0.0;
                    sa[j] = 0.0;
                }
                for (int64_t k = 0; alpha != 0.0 && k < K; ++k) {
                    double a = op_a(A, lda, transA, i, k);
                    const float* brow = bk + k * bld;
                    for (int64_t j = 0; j < N; ++j) {
                        double p = a * (double)brow[j];
                        s[j] += p;
                        sa[j] += fabs(p);
                    }
                }
                for (int64_t j = 0; j < N; ++j) {
                    double c = alpha * s[j];
                    if (beta != 0.0)
                        c += beta * (double)Cin[i * ldc + j];
                    cref[t * N + j] = c;
                    sabs[t * N + j] = sa[j];
                }
            }
        }
        free(s);
        free(sa);
    }
    free(bt);
    return status;
}

/* Number of OpenMP threads the loops above will use (for reporting). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
