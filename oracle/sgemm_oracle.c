/*
 * sgemm_oracle.c -- CPU oracle for the single-precision matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code with the GPU library.
 *
 * What it computes is the definition of the product as stated on the pages:
 *   page "CUDA算子优化(4)：矩阵乘法", section "矩阵乘法的数学定义":
 *     for A (M x K) and B (K x N), C (M x N) has C[i][j] equal to the sum over
 *     k = 0 .. K-1 of A[i][k] * B[k][j];
 *   page "CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结", §三 (the
 *     formula) and §四 (the serial CPU version: three nested loops i, j, k
 *     with the k loop innermost, one running sum per output element).
 * Storage is row-major with explicit leading dimensions (element (r, c) of
 * X sits at X[r*ldx + c]); the pages use dense rows, i.e. ld = row length.
 *
 * Readings where the pages leave a step open:
 *   - The sum is accumulated in double.  The pages accumulate in float; a
 *     product of two floats is exact in double, so the only rounding left is
 *     that of the running sum, about 1e-16 relative per term.
 *   - Alongside C it returns S[i][j] = sum_k |A[i][k]| * |B[k][j]|, the scale
 *     against which a GPU result is judged (|C_gpu - C| <= 5e-4*S + 1e-6;
 *     the 5e-4 is the tolerance the page "CUDA算子优化(4)：矩阵乘法" passes
 *     to its result check in both of its test programs).
 *   - K == 0 gives the empty sum, C = 0 and S = 0.
 *
 * The k order of every sum is 0, 1, ..., K-1, so the full-matrix and the
 * per-element entry points return bit-identical values for the same (i, j).
 *
 * The general form (oracle_sgemm_ex_f64) is the same definition with the
 * operands of the BLAS-style boundary that the pages compare against (their
 * cuBLAS baseline, page "CUDA算子优化(4)：矩阵乘法"):
 *     C_out[i][j] = alpha * sum_k opA[i][k] * opB[k][j] + beta * C_in[i][j]
 * where opA = A (M x K, A[i*lda + k]) or, transposed, the K x M array A read
 * as A[k*lda + i]; likewise opB = B (K x N, B[k*ldb + j]) or the N x K array
 * B read as B[j*ldb + k].  Readings (the pages never scale or accumulate):
 *   - beta == 0 means C_in is not read at all, so NaN or Inf there does not
 *     reach the result; alpha == 0 means A and B are not read (the BLAS
 *     convention).
 *   - The scale becomes S = |alpha| * sum_k |opA||opB| + |beta| * |C_in|; the
 *     two extra fp32 roundings of the scaling and the add stay far below
 *     5e-4 of it.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread sgemm_oracle.c -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>

/* One output element: the definition, term by term in k order. */
static void oracle_element(int64_t K, const float *A, int64_t lda,
                           const float *B, int64_t ldb, int64_t i, int64_t j,
                           double *c_out, double *s_out) {
    double c = 0.0;
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = (double)A[i * lda + k];
        double b = (double)B[k * ldb + j];
        c += a * b;
        s += fabs(a) * fabs(b);
    }
    *c_out = c;
    *s_out = s;
}

typedef struct {
    int64_t M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    double *C;
    int64_t ldc;
    double *S;
    int64_t lds;
    /* element-list mode */
    const int64_t *rows;
    const int64_t *cols;
    int64_t first, last;
} oracle_job;

static void *full_rows(void *arg) {
    oracle_job *j = (oracle_job *)arg;
    for (int64_t i = j->first; i < j->last; ++i)
        for (int64_t c = 0; c < j->N; ++c)
            oracle_element(j->K, j->A, j->lda, j->B, j->ldb, i, c,
                           &j->C[i * j->ldc + c], &j->S[i * j->lds + c]);
    return 0;
}

static void *listed_elements(void *arg) {
    oracle_job *j = (oracle_job *)arg;
    for (int64_t e = j->first; e < j->last; ++e)
        oracle_element(j->K, j->A, j->lda, j->B, j->ldb, j->rows[e], j->cols[e],
                       &j->C[e], &j->S[e]);
    return 0;
}

/* Split [0, count) statically over nthreads workers running fn. */
static void run_split(oracle_job proto, int64_t count, int nthreads,
                      void *(*fn)(void *)) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > count) nthreads = (int)count;
    oracle_job jobs[256];
    pthread_t tid[256];
    int started[256];
    int64_t chunk = (count + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].first = t * chunk;
        jobs[t].last = jobs[t].first + chunk < count ? jobs[t].first + chunk : count;
        started[t] = 0;
        if (jobs[t].first >= jobs[t].last) continue;
        if (t + 1 < nthreads && pthread_create(&tid[t], 0, fn, &jobs[t]) == 0)
            started[t] = 1;
        else
            fn(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t]) pthread_join(tid[t], 0);
}

static int bad_dims(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    return M < 0 || N < 0 || K < 0 || (K > 0 && lda < K) || (N > 0 && ldb < N);
}

/*
 * Full product: C[i*ldc + j] and S[i*lds + j] for all i < M, j < N.
 * Returns 0, or -1 on inconsistent sizes.
 */
int oracle_sgemm_f64(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda, const float *B, int64_t ldb,
                     double *C, int64_t ldc, double *S, int64_t lds,
                     int nthreads) {
    if (bad_dims(M, N, K, lda, ldb) || ldc < N || lds < N) return -1;
    if (M == 0 || N == 0) return 0;
    oracle_job proto = {M, N, K, A, lda, B, ldb, C, ldc, S, lds, 0, 0, 0, 0};
    run_split(proto, M, nthreads, full_rows);
    return 0;
}

/*
 * Listed elements: for e < count, C[e] and S[e] are element
 * (rows[e], cols[e]) of the product.  Used to check sampled outputs of
 * products too large to compute whole on the host.
 */
int oracle_sgemm_f64_elems(int64_t M, int64_t N, int64_t K,
                           const float *A, int64_t lda, const float *B, int64_t ldb,
                           int64_t count, const int64_t *rows, const int64_t *cols,
                           double *C, double *S, int nthreads) {
    if (bad_dims(M, N, K, lda, ldb) || count < 0) return -1;
    for (int64_t e = 0; e < count; ++e)
        if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N) return -1;
    if (count == 0) return 0;
    oracle_job proto = {M, N, K, A, lda, B, ldb, C, 0, S, 0, rows, cols, 0, 0};
    run_split(proto, count, nthreads, listed_elements);
    return 0;
}

/* ---- general form: alpha * op(A) op(B) + beta * C_in ---- */

typedef struct {
    int transa, transb;
    int64_t M, N, K;
    double alpha, beta;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    const float *Cin;
    int64_t ldcin;
    double *C;
    int64_t ldc;
    double *S;
    int64_t lds;
    const int64_t *rows; /* NULL: all of row i, else the listed elements */
    const int64_t *cols;
    int64_t first, last;
} oracle_ex_job;

/* Element (i, j) of the general form, the k sum in order 0 .. K-1. */
static void oracle_element_ex(const oracle_ex_job *p, int64_t i, int64_t j,
                              double *c_out, double *s_out) {
    double c = 0.0;
    double s = 0.0;
    if (p->alpha != 0.0) {
        for (int64_t k = 0; k < p->K; ++k) {
            double a = p->transa ? (double)p->A[k * p->lda + i] : (double)p->A[i * p->lda + k];
            double b = p->transb ? (double)p->B[j * p->ldb + k] : (double)p->B[k * p->ldb + j];
            c += a * b;
            s += fabs(a) * fabs(b);
        }
    }
    double out = p->alpha * c;
    double scale = fabs(p->alpha) * s;
    if (p->beta != 0.0) {
        double cin = (double)p->Cin[i * p->ldcin + j];
        out += p->beta * cin;
        scale += fabs(p->beta) * fabs(cin);
    }
    *c_out = out;
    *s_out = scale;
}

static void *ex_worker(void *arg) {
    oracle_ex_job *p = (oracle_ex_job *)arg;
    if (p->rows == 0) {
        for (int64_t i = p->first; i < p->last; ++i)
            for (int64_t j = 0; j < p->N; ++j)
                oracle_element_ex(p, i, j, &p->C[i * p->ldc + j], &p->S[i * p->lds + j]);
    } else {
        for (int64_t e = p->first; e < p->last; ++e)
            oracle_element_ex(p, p->rows[e], p->cols[e], &p->C[e], &p->S[e]);
    }
    return 0;
}

/*
 * General form.  With rows == NULL, C[i*ldc + j] and S[i*lds + j] for all
 * i < M, j < N; otherwise C[e] and S[e] for the count listed elements
 * (rows[e], cols[e]).  Cin may be NULL when beta == 0; A and B may be NULL
 * when alpha == 0 or K == 0.  Returns 0, or -1 on inconsistent arguments.
 */
int oracle_sgemm_ex_f64(int transa, int transb, int64_t M, int64_t N, int64_t K,
                        double alpha, const float *A, int64_t lda,
                        const float *B, int64_t ldb, double beta,
                        const float *Cin, int64_t ldcin,
                        int64_t count, const int64_t *rows, const int64_t *cols,
                        double *C, int64_t ldc, double *S, int64_t lds, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (K > 0 && alpha != 0.0) {
        if (lda < (transa ? M : K) || ldb < (transb ? K : N)) return -1;
        if (A == 0 || B == 0) return -1;
    }
    if (beta != 0.0 && (Cin == 0 || ldcin < N)) return -1;
    if (rows == 0 && (ldc < N || lds < N)) return -1;
    if (rows != 0)
        for (int64_t e = 0; e < count; ++e)
            if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N) return -1;
    int64_t units = rows == 0 ? M : count;
    if (units == 0 || N == 0) return 0;
    oracle_ex_job proto = {transa != 0, transb != 0, M, N, K, alpha, beta, A, lda, B, ldb,
                           Cin, ldcin, C, ldc, S, lds, rows, cols, 0, 0};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > units) nthreads = (int)units;
    oracle_ex_job jobs[256];
    pthread_t tid[256];
    int started[256];
    int64_t chunk = (units + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].first = t * chunk;
        jobs[t].last = jobs[t].first + chunk < units ? jobs[t].first + chunk : units;
        started[t] = 0;
        if (jobs[t].first >= jobs[t].last) continue;
        if (t + 1 < nthreads && pthread_create(&tid[t], 0, ex_worker, &jobs[t]) == 0)
            started[t] = 1;
        else
            ex_worker(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t]) pthread_join(tid[t], 0);
    return 0;
}
