/*
 * oracle_sgemm.c -- plain CPU reference for single-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header or constant with the
 * HIP path.
 *
 * What is computed
 * ----------------
 * Page "GEMM优化原理" (hatrix.site), section 问题定义, eq. 1, defines
 *     C = A x B,   C_ij = sum_{t=0}^{k-1} A_it * B_tj
 * with A m x k, B k x n and C m x n.  Page "GPU 访存与计算优化"
 * (aerisun.top), section "Naive GEMM 的重复读取", states the same sum.
 * The kernel signature printed on page "gemm优化" (blog.lightlisten.com),
 * section 性能分析, carries two float scalars next to the three matrices; they
 * are read as the usual scaling
 *     C_out_ij = alpha * S_ij + beta * C_in_ij,   S_ij = sum_t A_it * B_tj.
 * Storage is row-major (page aerisun.top, section "Shared Tiling 与 block 内
 * 复用", which assigns adjacent threads to adjacent columns of a row-major
 * operand) with a leading dimension per matrix:
 *     A_it = A[i*lda + t],  B_tj = B[t*ldb + j],  C_ij = C[i*ldc + j].
 * The _ex forms also take either operand stored transposed (the BLAS
 * op(X) = X^T; page "GEMM优化原理", section 基于 register 计算, discusses
 * reading an operand in transposed order):
 *     trans_a = 1:  A_it = A[t*lda + i]   (A stored k x m, lda >= m)
 *     trans_b = 1:  B_tj = B[j*ldb + t]   (B stored n x k, ldb >= k)
 * which is the same sum with other element addresses: the code below reads
 * A_it at A[i*sa_i + t*sa_t] and B_tj at B[t*sb_t + j*sb_j].
 *
 * How it is computed (nothing beyond the definition)
 * ---------------------------------------------------
 *  - every product A_it*B_tj of two floats is formed in double, where it is
 *    exact (24 + 24 significand bits fit in 53);
 *  - S_ij is summed in double over ascending t; G_ij = sum_t |A_it*B_tj| is
 *    summed alongside (the size of the terms, used by callers to state an
 *    error bound; page aerisun.top, section "Warp shuffle 的数据交换", notes
 *    that float addition is not associative, so results are compared with a
 *    tolerance rather than bitwise);
 *  - the result alpha*S_ij + beta*C_in_ij is formed in double and rounded to
 *    float once (round to nearest even, the C default).
 * Readings where the pages are silent:
 *  - beta == 0: C_in is not read at all (a NaN there does not reach C_out);
 *  - alpha == 0 or k == 0: A and B are not read and the S term is absent;
 *  - entries outside the logical m x k, k x n, m x n extents (the padding up
 *    to the leading dimension) are never read and never written.
 * The loop order i -> t -> j with a double row accumulator produces, for each
 * (i, j), exactly the ascending-t sum above; threads split the rows, so the
 * result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n, k;
    double alpha, beta;
    const float *A, *B;
    int64_t sa_i, sa_t;    /* A_it = A[i*sa_i + t*sa_t] */
    int64_t sb_t, sb_j;    /* B_tj = B[t*sb_t + j*sb_j] */
    int64_t ldc;
    float *C;              /* in/out, row-major with ldc */
    double *S, *G;         /* optional dense outputs, one row per computed row */
    const int64_t *rows;   /* rows to compute, or NULL for 0..nrows-1 */
    int64_t row_begin, row_end;  /* slice of the row list for this thread */
    int status;
} row_job;

/* One output row: S_ij and G_ij for all j, then the scaled, rounded result. */
static void one_row(const row_job *jb, int64_t slot, int64_t i,
                    double *acc, double *gacc)
{
    const int64_t n = jb->n, k = jb->k;
    const int use_ab = (k > 0 && jb->alpha != 0.0);
    for (int64_t j = 0; j < n; ++j) { acc[j] = 0.0; gacc[j] = 0.0; }
    if (use_ab) {
        for (int64_t t = 0; t < k; ++t) {
            const double a = (double)jb->A[i * jb->sa_i + t * jb->sa_t];
            const float *brow = jb->B + t * jb->sb_t;
            for (int64_t j = 0; j < n; ++j) {
                const double p = a * (double)brow[j * jb->sb_j];
                acc[j] += p;
                gacc[j] += fabs(p);
            }
        }
    }
    float *crow = jb->C + i * jb->ldc;
    for (int64_t j = 0; j < n; ++j) {
        double r = use_ab ? jb->alpha * acc[j] : 0.0;
        if (jb->beta != 0.0) r += jb->beta * (double)crow[j];
        crow[j] = (float)r;
    }
    if (jb->S) memcpy(jb->S + slot * n, acc, (size_t)n * sizeof(double));
    if (jb->G) memcpy(jb->G + slot * n, gacc, (size_t)n * sizeof(double));
}

static void *row_worker(void *arg)
{
    row_job *jb = (row_job *)arg;
    double *acc = (double *)malloc((size_t)(jb->n > 0 ? jb->n : 1) * sizeof(double));
    double *gacc = (double *)malloc((size_t)(jb->n > 0 ? jb->n : 1) * sizeof(double));
    if (!acc || !gacc) { free(acc); free(gacc); jb->status = -2; return NULL; }
    for (int64_t s = jb->row_begin; s < jb->row_end; ++s) {
        const int64_t i = jb->rows ? jb->rows[s] : s;
        one_row(jb, s, i, acc, gacc);
    }
    free(acc); free(gacc);
    jb->status = 0;
    return NULL;
}

/* Stored row widths: A is m x k (k x m transposed), B is k x n (n x k). */
static int bad_ld(int ta, int tb, int64_t m, int64_t n, int64_t k,
                  int64_t lda, int64_t ldb, int64_t ldc)
{
    const int64_t wa = ta ? m : k, wb = tb ? k : n;
    if ((ta != 0 && ta != 1) || (tb != 0 && tb != 1)) return 1;
    return lda < (wa > 1 ? wa : 1) || ldb < (wb > 1 ? wb : 1) || ldc < (n > 1 ? n : 1);
}

/*
 * oracle_sgemm_rows_ex: computes the output rows listed in `rows` (nrows
 * entries, each in [0, m)); rows == NULL means all rows 0..m-1 (nrows = m).
 * C is updated in place at those rows only.  S and G, when not NULL, receive
 * nrows x n dense doubles in the order of `rows`.  trans_a / trans_b (0 or 1)
 * select the stored forms described at the top of this file.
 * Returns 0 on success, -1 on a bad argument, -2 when memory runs out.
 */
int oracle_sgemm_rows_ex(int trans_a, int trans_b, int64_t m, int64_t n, int64_t k,
                         float alpha, const float *A, int64_t lda, const float *B, int64_t ldb,
                         float beta, float *C, int64_t ldc,
                         int64_t nrows, const int64_t *rows,
                         double *S, double *G, int nthreads)
{
    if (m < 0 || n < 0 || k < 0 || nrows < 0) return -1;
    if (!rows && nrows != m) return -1;
    if (nrows == 0 || n == 0) return 0;
    if (bad_ld(trans_a, trans_b, m, n, k, lda, ldb, ldc)) return -1;
    if (rows)
        for (int64_t s = 0; s < nrows; ++s)
            if (rows[s] < 0 || rows[s] >= m) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;

    row_job *jobs = (row_job *)calloc((size_t)nthreads, sizeof(row_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) { free(jobs); free(tids); return -2; }
    int rc = 0;
    for (int w = 0; w < nthreads; ++w) {
        row_job *jb = &jobs[w];
        jb->n = n; jb->k = k;
        jb->alpha = (double)alpha; jb->beta = (double)beta;
        jb->A = A; jb->B = B; jb->ldc = ldc;
        jb->sa_i = trans_a ? 1 : lda;
        jb->sa_t = trans_a ? lda : 1;
        jb->sb_t = trans_b ? 1 : ldb;
        jb->sb_j = trans_b ? ldb : 1;
        jb->C = C; jb->S = S; jb->G = G; jb->rows = rows;
        jb->row_begin = nrows * w / nthreads;
        jb->row_end = nrows * (w + 1) / nthreads;
        jb->status = -2;
    }
    int started = 0;
    for (int w = 1; w < nthreads; ++w) {
        if (pthread_create(&tids[w], NULL, row_worker, &jobs[w]) != 0) break;
        started = w;
    }
    /* rows of threads that could not be started are done here, in order */
    row_worker(&jobs[0]);
    for (int w = started + 1; w < nthreads; ++w) row_worker(&jobs[w]);
    for (int w = 1; w <= started; ++w) pthread_join(tids[w], NULL);
    for (int w = 0; w < nthreads; ++w) if (jobs[w].status != 0) rc = jobs[w].status;
    free(jobs); free(tids);
    return rc;
}

/*
 * oracle_sgemm_points_ex: single entries (ii[p], jj[p]) for p < npts,
 * computed as a dot product over ascending t -- the same sum, in the same
 * order, as the row form.  Results go to out[p] (float), S[p] and G[p]
 * (optional); C is only read (when beta != 0).
 */
int oracle_sgemm_points_ex(int trans_a, int trans_b, int64_t m, int64_t n, int64_t k,
                           float alpha, const float *A, int64_t lda, const float *B, int64_t ldb,
                           float beta, const float *C, int64_t ldc,
                           int64_t npts, const int64_t *ii, const int64_t *jj,
                           float *out, double *S, double *G)
{
    if (m < 0 || n < 0 || k < 0 || npts < 0) return -1;
    if (bad_ld(trans_a, trans_b, m, n, k, lda, ldb, ldc)) return -1;
    const int64_t sa_i = trans_a ? 1 : lda, sa_t = trans_a ? lda : 1;
    const int64_t sb_t = trans_b ? 1 : ldb, sb_j = trans_b ? ldb : 1;
    const double da = (double)alpha, db = (double)beta;
    const int use_ab = (k > 0 && alpha != 0.0f);
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t i = ii[p], j = jj[p];
        if (i < 0 || i >= m || j < 0 || j >= n) return -1;
        double s = 0.0, g = 0.0;
        if (use_ab) {
            for (int64_t t = 0; t < k; ++t) {
                const double prod = (double)A[i * sa_i + t * sa_t] * (double)B[t * sb_t + j * sb_j];
                s += prod;
                g += fabs(prod);
            }
        }
        double r = use_ab ? da * s : 0.0;
        if (db != 0.0) r += db * (double)C[i * ldc + j];
        out[p] = (float)r;
        if (S) S[p] = s;
        if (G) G[p] = g;
    }
    return 0;
}
