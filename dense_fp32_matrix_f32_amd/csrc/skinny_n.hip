// skinny_n.hip -- products with very few columns (N <= 8), e.g. a matrix times a vector.
//
// Mirror image of skinny.hip: with N small the intensity
// I = MNK / (2(MK + KN + MN)) (page "CUDA算子优化(4)：矩阵乘法", section "计算强度") is
// about N/2 flop per byte, so the product is bound by reading A once.  Each wave
// owns RW rows of A; its 64 lanes split K into 16-byte pieces (lane l reads
// k = 4l, 4l+256, ...), so every load instruction of the wave reads 1 KB of one
// row contiguously.  The few columns of B for those k are read once per lane and
// reused for all RW rows.  The 64 per-lane partial sums of each output are added
// by a fixed butterfly across the wave (lane 0's total is the result), so the
// result is reproducible run to run and no atomics are involved.
#include "internal.h"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SKINNY_N_MAX_COLS = 8;

__device__ __forceinline__ f32x4 load16_n(const float *p) {
    f32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// NR columns handled (N <= NR), RW rows per wave, 4 waves per work-group.
template <int NR, int RW>
__global__ __launch_bounds__(256) void skinny_n_kernel(int M, int N, int K,
                                                       const float *__restrict__ A, int64_t lda,
                                                       const float *__restrict__ B, int64_t ldb,
                                                       float *__restrict__ C, int64_t ldc,
                                                       float alpha, float beta) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * 4 + wave) * RW;

    const float *arow[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) arow[r] = A + (int64_t)min(row0 + r, M - 1) * lda;

    float acc[RW][NR];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int j = 0; j < NR; ++j) acc[r][j] = 0.0f;

    for (int k = 4 * lane; k < K; k += 256) {
        f32x4 a[RW];
        float b[4][NR];
        if (k + 3 < K) {
#pragma unroll
            for (int r = 0; r < RW; ++r) a[r] = load16_n(arow[r] + k);
            if (NR >= 4 && N == NR) {
                // Whole rows of B: NR/4 16-byte loads per k.
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int j4 = 0; j4 < NR / 4; ++j4) {
                        const f32x4 v = load16_n(B + (int64_t)(k + e) * ldb + 4 * j4);
                        b[e][4 * j4 + 0] = v.x;
                        b[e][4 * j4 + 1] = v.y;
                        b[e][4 * j4 + 2] = v.z;
                        b[e][4 * j4 + 3] = v.w;
                    }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int j = 0; j < NR; ++j)
                        b[e][j] = B[(int64_t)(k + e) * ldb + min(j, N - 1)];
            }
        } else {
            // Last partial piece of the row: terms with k >= K are zero.
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                a[r].x = arow[r][k];
                a[r].y = k + 1 < K ? arow[r][k + 1] : 0.0f;
                a[r].z = k + 2 < K ? arow[r][k + 2] : 0.0f;
                a[r].w = k + 3 < K ? arow[r][k + 3] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int j = 0; j < NR; ++j)
                    b[e][j] = k + e < K ? B[(int64_t)(k + e) * ldb + min(j, N - 1)] : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                acc[r][j] = fmaf(a[r].x, b[0][j], acc[r][j]);
                acc[r][j] = fmaf(a[r].y, b[1][j], acc[r][j]);
                acc[r][j] = fmaf(a[r].z, b[2][j], acc[r][j]);
                acc[r][j] = fmaf(a[r].w, b[3][j], acc[r][j]);
            }
    }

    // Butterfly over the 64 lanes, the same pairing for every output.
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int d = 32; d > 0; d >>= 1) acc[r][j] += __shfl_xor(acc[r][j], d, 64);

    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
            if (row0 + r < M)
#pragma unroll
                for (int j = 0; j < NR; ++j)
                    if (j < N) {
                        float *dst = C + (int64_t)(row0 + r) * ldc + j;
                        *dst = epilogue(acc[r][j], alpha, beta, dst);
                    }
    }
}

template <int NR>
static hipError_t launch_cols(const Problem &p, hipStream_t s) {
    // More rows per wave re-use each loaded row of B more often.
    constexpr int RW = NR <= 2 ? 4 : 8;
    const int64_t groups = (p.M + 4 * RW - 1) / (4 * RW);
    if (groups > INT32_MAX) return hipErrorInvalidValue;
    return launch(skinny_n_kernel<NR, RW>, dim3((unsigned)groups), dim3(256), 0, s, p.M, p.N, p.K,
                  p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.alpha, p.beta);
}

hipError_t launch_skinny_n(const Problem &p, hipStream_t s) {
    // More than 8 columns: one pass per group of 8 columns.
    for (int c0 = 0; c0 < p.N; c0 += SKINNY_N_MAX_COLS) {
        Problem q = p;
        q.N = p.N - c0 < SKINNY_N_MAX_COLS ? p.N - c0 : SKINNY_N_MAX_COLS;
        q.B = p.B + c0;
        q.C = p.C + c0;
        hipError_t e;
        if (q.N == 1) e = launch_cols<1>(q, s);
        else if (q.N == 2) e = launch_cols<2>(q, s);
        else if (q.N <= 4) e = launch_cols<4>(q, s);
        else e = launch_cols<8>(q, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sgemm
