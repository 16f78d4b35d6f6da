// sgemm_api.hip -- the C ABI of include/sgemm_f32.h: argument validation on the
// host (before any HIP call), choice of kernel, and launch on the caller's stream.
#include "sgemm_f32.h"

#include "internal.h"

using sgemm::Problem;

namespace {

// Byte extent [lo, hi) of a rows x cols row-major array with row stride ld.
struct Extent {
    uintptr_t lo, hi;
};

Extent extent(const void *p, int64_t rows, int64_t cols, int64_t ld) {
    const uintptr_t lo = (uintptr_t)p;
    return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * (int64_t)sizeof(float))};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

int at_least_one(int x) { return x > 1 ? x : 1; }

// hipSuccess if the arguments describe a valid C = alpha*op(A)*op(B) + beta*C,
// else hipErrorInvalidValue.  A and B are read only when alpha != 0 and K > 0.
hipError_t validate(int transa, int transb, int M, int N, int K, float alpha, const float *A,
                    int lda, const float *B, int ldb, const float *C, int ldc) {
    if ((transa != SGEMM_F32_OP_N && transa != SGEMM_F32_OP_T) ||
        (transb != SGEMM_F32_OP_N && transb != SGEMM_F32_OP_T))
        return hipErrorInvalidValue;
    if (M < 0 || N < 0 || K < 0) return hipErrorInvalidValue;
    if (lda < at_least_one(transa ? M : K) || ldb < at_least_one(transb ? K : N) ||
        ldc < at_least_one(N))
        return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    if (C == nullptr) return hipErrorInvalidValue;
    if (K == 0 || alpha == 0.0f) return hipSuccess;
    if (A == nullptr || B == nullptr) return hipErrorInvalidValue;
    const Extent c = extent(C, M, N, ldc);
    const Extent a = transa ? extent(A, K, M, lda) : extent(A, M, K, lda);
    const Extent b = transb ? extent(B, N, K, ldb) : extent(B, K, N, ldb);
    if (overlaps(c, a) || overlaps(c, b)) return hipErrorInvalidValue;
    return hipSuccess;
}

// Untransposed products with few rows or few columns stream one operand and are
// bound by memory, so the streaming kernels win; everything else goes to the
// matrix cores.
int choose(int transa, int transb, int M, int N, int K) {
    (void)K;
    if (transa == SGEMM_F32_OP_N && transb == SGEMM_F32_OP_N) {
        if (M <= 8) return SGEMM_F32_ALGO_SKINNY;
        if (N <= 8) return SGEMM_F32_ALGO_SKINNY_N;
    }
    return SGEMM_F32_ALGO_MFMA;
}

bool handles_transposes(int algo) {
    return algo == SGEMM_F32_ALGO_AUTO || algo == SGEMM_F32_ALGO_NAIVE ||
           algo == SGEMM_F32_ALGO_LDS_TILED || algo == SGEMM_F32_ALGO_MFMA;
}

Problem problem(int transa, int transb, int M, int N, int K, float alpha, const float *A,
                int lda, const float *B, int ldb, float beta, float *C, int ldc) {
    Problem p{M, N, K, A, lda, B, ldb, C, ldc};
    p.ta = transa == SGEMM_F32_OP_T;
    p.tb = transb == SGEMM_F32_OP_T;
    p.alpha = alpha;
    p.beta = beta;
    return p;
}

// Validation and the product-free cases shared by the entry points.  Returns
// true with *status set when nothing is left to launch.
bool trivial(int transa, int transb, int M, int N, int K, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream,
             hipError_t *status) {
    *status = validate(transa, transb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (*status != hipSuccess) return true;
    if (M == 0 || N == 0) return true;
    if (K == 0 || alpha == 0.0f) {
        *status = sgemm::launch_scale(
            problem(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc), stream);
        return true;
    }
    return false;
}

}  // namespace

extern "C" const char *sgemm_f32_algo_name(int algo) {
    switch (algo) {
    case SGEMM_F32_ALGO_AUTO: return "auto";
    case SGEMM_F32_ALGO_NAIVE: return "naive";
    case SGEMM_F32_ALGO_LDS_TILED: return "lds_tiled";
    case SGEMM_F32_ALGO_VALU_REGBLOCK: return "valu_regblock";
    case SGEMM_F32_ALGO_MFMA: return "mfma";
    case SGEMM_F32_ALGO_SKINNY: return "skinny";
    case SGEMM_F32_ALGO_SKINNY_N: return "skinny_n";
    case SGEMM_F32_ALGO_BF16X6: return "bf16x6";
    default: return "invalid";
    }
}

extern "C" int sgemm_f32_select(int M, int N, int K, const float *A, int lda, const float *B,
                                int ldb, const float *C, int ldc) {
    if (validate(SGEMM_F32_OP_N, SGEMM_F32_OP_N, M, N, K, 1.0f, A, lda, B, ldb, C, ldc) !=
        hipSuccess)
        return -1;
    return choose(SGEMM_F32_OP_N, SGEMM_F32_OP_N, M, N, K);
}

extern "C" hipError_t sgemm_f32_ex_algo(int transa, int transb, int M, int N, int K, float alpha,
                                        const float *A, int lda, const float *B, int ldb,
                                        float beta, float *C, int ldc, hipStream_t stream,
                                        int algo) {
    if (algo < 0 || algo >= SGEMM_F32_ALGO_COUNT) return hipErrorInvalidValue;
    if ((transa == SGEMM_F32_OP_T || transb == SGEMM_F32_OP_T) && !handles_transposes(algo))
        return hipErrorInvalidValue;
    hipError_t st;
    if (trivial(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, &st))
        return st;
    const Problem p = problem(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    if (algo == SGEMM_F32_ALGO_AUTO) algo = choose(transa, transb, M, N, K);
    switch (algo) {
    case SGEMM_F32_ALGO_NAIVE: return sgemm::launch_naive(p, stream);
    case SGEMM_F32_ALGO_LDS_TILED: return sgemm::launch_lds_tiled(p, stream);
    case SGEMM_F32_ALGO_VALU_REGBLOCK: return sgemm::launch_valu_regblock(p, stream);
    case SGEMM_F32_ALGO_MFMA: return sgemm::launch_mfma(p, stream);
    case SGEMM_F32_ALGO_SKINNY: return sgemm::launch_skinny(p, stream);
    case SGEMM_F32_ALGO_SKINNY_N: return sgemm::launch_skinny_n(p, stream);
    case SGEMM_F32_ALGO_BF16X6: return sgemm::launch_split(p, stream);
    default: return hipErrorInvalidValue;
    }
}

extern "C" hipError_t sgemm_f32_ex(int transa, int transb, int M, int N, int K, float alpha,
                                   const float *A, int lda, const float *B, int ldb, float beta,
                                   float *C, int ldc, hipStream_t stream) {
    return sgemm_f32_ex_algo(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                             SGEMM_F32_ALGO_AUTO);
}

extern "C" hipError_t sgemm_f32_algo(int M, int N, int K, const float *A, int lda,
                                     const float *B, int ldb, float *C, int ldc,
                                     hipStream_t stream, int algo) {
    return sgemm_f32_ex_algo(SGEMM_F32_OP_N, SGEMM_F32_OP_N, M, N, K, 1.0f, A, lda, B, ldb, 0.0f,
                             C, ldc, stream, algo);
}

extern "C" hipError_t sgemm_f32(int M, int N, int K, const float *A, int lda, const float *B,
                                int ldb, float *C, int ldc, hipStream_t stream) {
    return sgemm_f32_algo(M, N, K, A, lda, B, ldb, C, ldc, stream, SGEMM_F32_ALGO_AUTO);
}

extern "C" hipError_t sgemm_f32_colmajor(int transa, int transb, int M, int N, int K,
                                         float alpha, const float *A, int lda, const float *B,
                                         int ldb, float beta, float *C, int ldc,
                                         hipStream_t stream) {
    // A column-major array is the row-major array of its transpose, so
    // C^T = alpha*op(B)^T*op(A)^T + beta*C^T in row-major terms.
    return sgemm_f32_ex(transb, transa, N, M, K, alpha, B, ldb, A, lda, beta, C, ldc, stream);
}

extern "C" int sgemm_f32_mfma_tiles(void) { return sgemm::mfma_tile_count(); }

extern "C" const char *sgemm_f32_mfma_tile_name(int tile) { return sgemm::mfma_tile_name(tile); }

extern "C" int sgemm_f32_mfma_select(int M, int N, int K, int compute_units) {
    if (M < 0 || N < 0 || K < 0) return -1;
    return sgemm::mfma_select(M, N, K, compute_units);
}

extern "C" hipError_t sgemm_f32_ex_mfma_tile(int transa, int transb, int M, int N, int K,
                                             float alpha, const float *A, int lda,
                                             const float *B, int ldb, float beta, float *C,
                                             int ldc, hipStream_t stream, int tile) {
    if (tile < 0 || tile >= sgemm::mfma_tile_count()) return hipErrorInvalidValue;
    hipError_t st;
    if (trivial(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, &st))
        return st;
    return sgemm::launch_mfma_tile(
        problem(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc), stream, tile);
}

extern "C" hipError_t sgemm_f32_mfma_tile(int M, int N, int K, const float *A, int lda,
                                          const float *B, int ldb, float *C, int ldc,
                                          hipStream_t stream, int tile) {
    return sgemm_f32_ex_mfma_tile(SGEMM_F32_OP_N, SGEMM_F32_OP_N, M, N, K, 1.0f, A, lda, B, ldb,
                                  0.0f, C, ldc, stream, tile);
}
