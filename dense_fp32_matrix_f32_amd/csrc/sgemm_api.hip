// sgemm_api.hip -- the C ABI of include/sgemm_f32.h: argument validation on the
// host (before any HIP call), choice of kernel, and launch on the caller's stream.
#include "sgemm_f32.h"

#include "internal.h"

using sgemm::Problem;

namespace {

// Byte extent [lo, hi) of a rows x cols row-major operand with row stride ld.
struct Extent {
    uintptr_t lo, hi;
};

Extent extent(const void *p, int64_t rows, int64_t cols, int64_t ld) {
    const uintptr_t lo = (uintptr_t)p;
    return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * (int64_t)sizeof(float))};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

// hipSuccess if the arguments are a valid product, else hipErrorInvalidValue.
hipError_t validate(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                    const float *C, int ldc) {
    if (M < 0 || N < 0 || K < 0) return hipErrorInvalidValue;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    if (C == nullptr) return hipErrorInvalidValue;
    if (K == 0) return hipSuccess;
    if (A == nullptr || B == nullptr) return hipErrorInvalidValue;
    const Extent c = extent(C, M, N, ldc);
    if (overlaps(c, extent(A, M, K, lda)) || overlaps(c, extent(B, K, N, ldb)))
        return hipErrorInvalidValue;
    return hipSuccess;
}

// Few rows or few columns: the product streams one operand and is bound by
// memory, so the streaming kernels win; everything else goes to matrix cores.
int choose(int M, int N, int K) {
    (void)K;
    if (M <= 8) return SGEMM_F32_ALGO_SKINNY;
    if (N <= 8) return SGEMM_F32_ALGO_SKINNY_N;
    return SGEMM_F32_ALGO_MFMA;
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
    default: return "invalid";
    }
}

extern "C" int sgemm_f32_select(int M, int N, int K, const float *A, int lda, const float *B,
                                int ldb, const float *C, int ldc) {
    if (validate(M, N, K, A, lda, B, ldb, C, ldc) != hipSuccess) return -1;
    return choose(M, N, K);
}

extern "C" hipError_t sgemm_f32_algo(int M, int N, int K, const float *A, int lda,
                                     const float *B, int ldb, float *C, int ldc,
                                     hipStream_t stream, int algo) {
    if (algo < 0 || algo >= SGEMM_F32_ALGO_COUNT) return hipErrorInvalidValue;
    const hipError_t v = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (v != hipSuccess) return v;
    if (M == 0 || N == 0) return hipSuccess;
    const Problem p{M, N, K, A, lda, B, ldb, C, ldc};
    if (K == 0) return sgemm::launch_zero_fill(p, stream);
    if (algo == SGEMM_F32_ALGO_AUTO) algo = choose(M, N, K);
    switch (algo) {
    case SGEMM_F32_ALGO_NAIVE: return sgemm::launch_naive(p, stream);
    case SGEMM_F32_ALGO_LDS_TILED: return sgemm::launch_lds_tiled(p, stream);
    case SGEMM_F32_ALGO_VALU_REGBLOCK: return sgemm::launch_valu_regblock(p, stream);
    case SGEMM_F32_ALGO_MFMA: return sgemm::launch_mfma(p, stream);
    case SGEMM_F32_ALGO_SKINNY: return sgemm::launch_skinny(p, stream);
    case SGEMM_F32_ALGO_SKINNY_N: return sgemm::launch_skinny_n(p, stream);
    default: return hipErrorInvalidValue;
    }
}

extern "C" hipError_t sgemm_f32(int M, int N, int K, const float *A, int lda, const float *B,
                                int ldb, float *C, int ldc, hipStream_t stream) {
    return sgemm_f32_algo(M, N, K, A, lda, B, ldb, C, ldc, stream, SGEMM_F32_ALGO_AUTO);
}

extern "C" int sgemm_f32_mfma_tiles(void) { return sgemm::mfma_tile_count(); }

extern "C" const char *sgemm_f32_mfma_tile_name(int tile) { return sgemm::mfma_tile_name(tile); }

extern "C" int sgemm_f32_mfma_select(int M, int N, int K, int compute_units) {
    if (M < 0 || N < 0 || K < 0) return -1;
    return sgemm::mfma_select(M, N, K, compute_units);
}

extern "C" hipError_t sgemm_f32_mfma_tile(int M, int N, int K, const float *A, int lda,
                                          const float *B, int ldb, float *C, int ldc,
                                          hipStream_t stream, int tile) {
    if (tile < 0 || tile >= sgemm::mfma_tile_count()) return hipErrorInvalidValue;
    const hipError_t v = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (v != hipSuccess) return v;
    if (M == 0 || N == 0) return hipSuccess;
    const Problem p{M, N, K, A, lda, B, ldb, C, ldc};
    if (K == 0) return sgemm::launch_zero_fill(p, stream);
    return sgemm::launch_mfma_tile(p, stream, tile);
}
