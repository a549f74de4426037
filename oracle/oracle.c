/*
 * Reference SGEMM on the host, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library
 * shares no code, header, table or constant with this file, and nothing on
 * the product path may call it.
 *
 * What it computes (the plain definition, nothing else):
 *   C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 * for row-major A (M x K, leading dimension lda) and B (K x N, leading
 * dimension ldb).  This is the matrix-multiplication definition stated in
 * "CUDA 算子优化：GEMM" (llm-tech.com.cn), section "矩阵乘法", and in
 * "GEMM from naive to tiled" (arganzheng.life), section 一.2 (notation:
 * C = A·B, all row-major, FP32 operands).
 *
 * Precision: every fp32 x fp32 product is exact in binary64 (24 + 24 <= 53
 * significand bits), so the only rounding is in the fp64 additions, taken
 * in ascending k for every (i, j).  The loop order is row i, then k, then j,
 * with a row accumulator: each element still sums its products in
 * ascending k, so the result is bit-for-bit that of the textbook i-j-k
 * triple loop.  Build without -ffast-math (no reassociation).
 *
 * The denominator D[i][j] = sum_k |A[i][k]| * |B[k][j]| is the scale the
 * acceptance bound is measured against: |C_gpu - C| <= tol * D.
 *
 * Threads: rows are independent, so the OpenMP split over rows does not
 * change any result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the following calls use (n >= 1); results do not depend on it. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Full product.  C (M x N, leading dimension ldc) receives the fp64 sums.
 * D, when not NULL, receives sum_k |A||B| with leading dimension ldd.
 * Returns 0 on success, -1 on bad arguments, -2 if scratch allocation fails.
 */
int oracle_sgemm(int64_t M, int64_t N, int64_t K,
                 const float* A, int64_t lda,
                 const float* B, int64_t ldb,
                 double* C, int64_t ldc,
                 double* D, int64_t ldd) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (C == NULL || ldc < N) return -1;
    if (D != NULL && ldd < N) return -1;
    if (K > 0 && (A == NULL || B == NULL || lda < K || ldb < N)) return -1;
    int failed = 0;
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)N * sizeof(double));
        double* aacc = (D != NULL) ? (double*)malloc((size_t)N * sizeof(double)) : NULL;
        if (acc == NULL || (D != NULL && aacc == NULL)) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            if (acc == NULL || (D != NULL && aacc == NULL)) continue;
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            if (aacc) for (int64_t j = 0; j < N; ++j) aacc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = (double)A[i * lda + k];
                const float* brow = B + k * ldb;
                for (int64_t j = 0; j < N; ++j) acc[j] += a * (double)brow[j];
                if (aacc) {
                    const double aa = fabs(a);
                    for (int64_t j = 0; j < N; ++j) aacc[j] += aa * fabs((double)brow[j]);
                }
            }
            memcpy(C + i * ldc, acc, (size_t)N * sizeof(double));
            if (aacc) memcpy(D + i * ldd, aacc, (size_t)N * sizeof(double));
        }
        free(acc);
        free(aacc);
    }
    return failed ? -2 : 0;
}

/*
 * The library-call form: C = alpha * op(A) * op(B) + beta * Cin, row-major,
 * with op(X) = X or its transpose.  This is the operation behind the BLAS
 * call that "GEMM from naive to tiled" (arganzheng.life), section 二.2,
 * follows from torch.matmul down to (transa, transb, m, n, k, alpha, A, lda,
 * B, ldb, beta, C, ldc), with the row-major reading of section 一.2:
 *   op(A)[i][k] = trans_a ? A[k * lda + i] : A[i * lda + k]   (A stored K x M or M x K)
 *   op(B)[k][j] = trans_b ? B[j * ldb + k] : B[k * ldb + j]   (B stored N x K or K x N)
 *   C[i][j] = alpha * sum_{k<K} op(A)[i][k] op(B)[k][j] + beta * Cin[i][j]
 * The sum is taken in fp64 in ascending k, as in oracle_sgemm.  The BLAS
 * conventions for the scalars are kept: with beta == 0, Cin is not read (so
 * NaN there does not propagate); with alpha == 0 or K == 0, A and B are not
 * read and C = beta * Cin.
 * D (when not NULL) receives the error scale
 *   |alpha| * sum_k |op(A)[i][k]| |op(B)[k][j]| + |beta| * |Cin[i][j]|
 * (each term only where it is computed).
 * Returns 0 on success, -1 on bad arguments, -2 if scratch allocation fails.
 */
int oracle_gemm(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, double alpha,
                const float* A, int64_t lda, const float* B, int64_t ldb, double beta,
                const float* Cin, int64_t ldcin, double* C, int64_t ldc, double* D, int64_t ldd) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (C == NULL || ldc < N) return -1;
    if (D != NULL && ldd < N) return -1;
    const int use_ab = alpha != 0.0 && K > 0;
    if (use_ab) {
        if (A == NULL || B == NULL) return -1;
        if (lda < (trans_a ? M : K) || ldb < (trans_b ? K : N)) return -1;
    }
    if (beta != 0.0 && (Cin == NULL || ldcin < N)) return -1;
    int failed = 0;
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)N * sizeof(double));
        double* aacc = (double*)malloc((size_t)N * sizeof(double));
        if (acc == NULL || aacc == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            if (acc == NULL || aacc == NULL) continue;
            for (int64_t j = 0; j < N; ++j) acc[j] = aacc[j] = 0.0;
            if (use_ab) {
                for (int64_t k = 0; k < K; ++k) {
                    const double a = (double)(trans_a ? A[k * lda + i] : A[i * lda + k]);
                    for (int64_t j = 0; j < N; ++j) {
                        const double b = (double)(trans_b ? B[j * ldb + k] : B[k * ldb + j]);
                        acc[j] += a * b;
                        aacc[j] += fabs(a) * fabs(b);
                    }
                }
            }
            for (int64_t j = 0; j < N; ++j) {
                double c = use_ab ? alpha * acc[j] : 0.0;
                double d = use_ab ? fabs(alpha) * aacc[j] : 0.0;
                if (beta != 0.0) {
                    const double cin = (double)Cin[i * ldcin + j];
                    c += beta * cin;
                    d += fabs(beta) * fabs(cin);
                }
                C[i * ldc + j] = c;
                if (D != NULL) D[i * ldd + j] = d;
            }
        }
        free(acc);
        free(aacc);
    }
    return failed ? -2 : 0;
}

/*
 * Selected entries only: for each t < count, c_out[t] = C[rows[t]][cols[t]]
 * and (when d_out is not NULL) d_out[t] = D[rows[t]][cols[t]], each a dot
 * product summed in ascending k.  Lets a full-size product be checked on
 * sampled outputs.  Returns -1 if an index is out of range.
 */
int oracle_sgemm_entries(int64_t M, int64_t N, int64_t K,
                         const float* A, int64_t lda,
                         const float* B, int64_t ldb,
                         int64_t count, const int64_t* rows, const int64_t* cols,
                         double* c_out, double* d_out) {
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (count == 0) return 0;
    if (rows == NULL || cols == NULL || c_out == NULL) return -1;
    if (K > 0 && (A == NULL || B == NULL || lda < K || ldb < N)) return -1;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = (double)A[i * lda + k] * (double)B[k * ldb + j];
            s += p;
            sa += fabs(p);
        }
        c_out[t] = s;
        if (d_out) d_out[t] = sa;
    }
    return 0;
}

/*
 * y[i] = sum_k op(A[i][k]) * x[k] in fp64, with op the identity, or the
 * absolute value of both factors when absolute != 0.  Used for the
 * associativity property (AB)x = A(Bx) at full size: A(Bx) costs O(MK + KN)
 * where AB costs O(MNK), and |A|(|B||x|) bounds the error of (AB)x.
 */
int oracle_gemv(int64_t M, int64_t K, const float* A, int64_t lda,
                const double* x, double* y, int absolute) {
    if (M < 0 || K < 0) return -1;
    if (M == 0) return 0;
    if (y == NULL) return -1;
    if (K > 0 && (A == NULL || x == NULL || lda < K)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            s += absolute ? fabs(a) * fabs(x[k]) : a * x[k];
        }
        y[i] = s;
    }
    return 0;
}

/*
 * Round fp64 results to binary32, round-to-nearest-even (the C cast under
 * the default rounding mode): the fp32 value nearest the oracle's sum.
 */
void oracle_round_to_f32(int64_t n, const double* in, float* out) {
    for (int64_t t = 0; t < n; ++t) out[t] = (float)in[t];
}
