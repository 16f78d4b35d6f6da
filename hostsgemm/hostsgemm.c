/*
 * hostsgemm.c -- a cache-blocked, multi-threaded fp32 matrix product on the host
 * CPU: the stronger host baseline next to the oracle.
 *
 * The page "CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结" (§四) measures a
 * serial triple loop and notes that it uses a single core.  This is the same
 * product, C = A·B in fp32 with row-major A (M x K), B (K x N), C (M x N) and
 * element strides, arranged for a multi-core CPU in the usual way:
 *   - C is split into row ranges, one per thread (no synchronisation);
 *   - k runs in panels of KC; per panel a thread packs NC columns of B into
 *     NR-wide strips and MC rows of A into MR-tall strips, both contiguous in k;
 *   - a register-blocked MR x NR micro-kernel accumulates the panel's outer
 *     products in fp32 (vector fused multiply-adds) and adds them to C.
 * Partial strips at the edges are zero-padded in the packed copies and only
 * the valid part of C is written.  It is a baseline for timing, not a
 * reference: results are checked against the oracle, within its tolerance.
 *
 * Build: gcc -O3 -march=x86-64-v3 -fPIC -shared -pthread hostsgemm.c
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MR 6
#define NR 16
#define MC 96
#define KC 256
#define NC 2048

typedef float v8 __attribute__((vector_size(32)));

static inline v8 load8(const float *p) {
    v8 v;
    memcpy(&v, p, sizeof(v));
    return v;
}

static inline void store8(float *p, v8 v) { memcpy(p, &v, sizeof(v)); }

static inline v8 splat(float x) { return (v8){x, x, x, x, x, x, x, x}; }

/* acc[MR][NR] = sum over kc of Ap[k][r] * Bp[k][c] (packed strips). */
static void micro_kernel(int kc, const float *Ap, const float *Bp, float *acc) {
    v8 c[MR][2];
    for (int r = 0; r < MR; ++r) c[r][0] = c[r][1] = splat(0.0f);
    for (int k = 0; k < kc; ++k) {
        const v8 b0 = load8(Bp + k * NR), b1 = load8(Bp + k * NR + 8);
        for (int r = 0; r < MR; ++r) {
            const v8 a = splat(Ap[k * MR + r]);
            c[r][0] += a * b0;
            c[r][1] += a * b1;
        }
    }
    for (int r = 0; r < MR; ++r) {
        store8(acc + r * NR, c[r][0]);
        store8(acc + r * NR + 8, c[r][1]);
    }
}

typedef struct {
    int64_t M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
    int64_t row0, row1;
    int status;
} job;

static void *run(void *arg) {
    job *j = (job *)arg;
    float *Bp = aligned_alloc(64, sizeof(float) * (size_t)KC * NC);
    float *Ap = aligned_alloc(64, sizeof(float) * (size_t)KC * MC);
    if (!Bp || !Ap) {
        free(Bp);
        free(Ap);
        j->status = -1;
        return 0;
    }
    float acc[MR * NR];
    for (int64_t i = j->row0; i < j->row1; ++i)
        for (int64_t c = 0; c < j->N; ++c) j->C[i * j->ldc + c] = 0.0f;
    for (int64_t n0 = 0; n0 < j->N; n0 += NC) {
        const int64_t nc = j->N - n0 < NC ? j->N - n0 : NC;
        for (int64_t k0 = 0; k0 < j->K; k0 += KC) {
            const int kc = (int)(j->K - k0 < KC ? j->K - k0 : KC);
            /* pack B[k0 : k0+kc, n0 : n0+nc] into NR-wide strips */
            for (int64_t s = 0; s < nc; s += NR) {
                float *dst = Bp + s * kc;
                for (int k = 0; k < kc; ++k) {
                    const float *src = j->B + (k0 + k) * j->ldb + n0 + s;
                    for (int c = 0; c < NR; ++c) dst[k * NR + c] = s + c < nc ? src[c] : 0.0f;
                }
            }
            for (int64_t m0 = j->row0; m0 < j->row1; m0 += MC) {
                const int64_t mc = j->row1 - m0 < MC ? j->row1 - m0 : MC;
                /* pack A[m0 : m0+mc, k0 : k0+kc] into MR-tall strips */
                for (int64_t s = 0; s < mc; s += MR) {
                    float *dst = Ap + s * kc;
                    for (int r = 0; r < MR; ++r) {
                        const float *src = j->A + (m0 + s + r) * j->lda + k0;
                        const int valid = s + r < mc;
                        for (int k = 0; k < kc; ++k) dst[k * MR + r] = valid ? src[k] : 0.0f;
                    }
                }
                for (int64_t s = 0; s < mc; s += MR) {
                    for (int64_t t = 0; t < nc; t += NR) {
                        micro_kernel(kc, Ap + s * kc, Bp + t * kc, acc);
                        const int64_t rows = mc - s < MR ? mc - s : MR;
                        const int64_t cols = nc - t < NR ? nc - t : NR;
                        for (int64_t r = 0; r < rows; ++r) {
                            float *dst = j->C + (m0 + s + r) * j->ldc + n0 + t;
                            for (int64_t c = 0; c < cols; ++c) dst[c] += acc[r * NR + c];
                        }
                    }
                }
            }
        }
    }
    free(Bp);
    free(Ap);
    j->status = 0;
    return 0;
}

/*
 * C = A·B on `nthreads` threads (row ranges of C).  Returns 0, or -1 on
 * inconsistent sizes or when memory for the packed panels is not available.
 */
int host_sgemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
               int64_t ldb, float *C, int64_t ldc, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || (K > 0 && lda < K) || (N > 0 && (ldb < N || ldc < N)))
        return -1;
    if (M == 0 || N == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > M) nthreads = (int)M;
    job jobs[256];
    pthread_t tid[256];
    int started[256];
    /* row ranges in multiples of MR so that strips stay whole */
    const int64_t strips = (M + MR - 1) / MR;
    const int64_t per = (strips + nthreads - 1) / nthreads;
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        const int64_t r0 = t * per * MR, r1 = (t + 1) * per * MR;
        jobs[t] = (job){M, N, K, A, lda, B, ldb, C, ldc, r0 < M ? r0 : M, r1 < M ? r1 : M, 0};
        started[t] = 0;
        if (jobs[t].row0 >= jobs[t].row1) continue;
        if (t + 1 < nthreads && pthread_create(&tid[t], 0, run, &jobs[t]) == 0)
            started[t] = 1;
        else
            run(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) {
        if (started[t]) pthread_join(tid[t], 0);
        if (jobs[t].row0 < jobs[t].row1 && jobs[t].status != 0) rc = -1;
    }
    return rc;
}
