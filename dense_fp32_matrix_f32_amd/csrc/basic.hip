// basic.hip -- the first two rungs of the kernel ladder and the product-free
// scaling of C.
//
// Rung 0 (naive) and rung 1 (LDS-tiled) are the two GPU designs that the pages
// build: one thread per output element reading A and B straight from global
// memory, then the same mapping with A and B staged tile by tile in on-chip
// memory.  They are kept as reference points for the faster rungs and accept
// every shape and either storage order of each operand.
#include "internal.h"

namespace sgemm {


// ---------------------------------------------------------------------------
// No product (K == 0, the empty sum, or alpha == 0): C = beta*C, and C = 0
// without reading it when beta == 0.
__global__ __launch_bounds__(256) void scale_kernel(int M, int N, float *__restrict__ C,
                                                    int64_t ldc, float beta) {
    const int64_t total = (int64_t)M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t i = e / N, j = e - i * N;
        float *c = C + i * ldc + j;
        *c = beta == 0.0f ? 0.0f : beta * *c;
    }
}

hipError_t launch_scale(const Problem &p, hipStream_t s) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    return launch(scale_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p.M, p.N, p.C, p.ldc,
                  p.beta);
}

// ---------------------------------------------------------------------------
// Split-k: C = alpha * (sum of the S planes) + beta * C, the planes (M x N, row
// stride N) added in an order fixed by (M, N, S) alone, so the result does not
// depend on which work-group finished first.  A work-group covers E = 256/G
// consecutive elements with G groups of work-items: group g adds planes
// [g*S/G, (g+1)*S/G) in order, then group 0 adds the G partial sums in order.
// G > 1 spreads small outputs (128 x 128 is 64 work-groups of 256 elements)
// over more CUs and shortens each work-item's chain of plane loads.  Loads are
// issued in batches of 16 (then 4) before they are added, so several reads are
// in flight per work-item.
template <int G>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(int M, int N, int S,
                                                            const float *__restrict__ ws,
                                                            float *__restrict__ C, int64_t ldc,
                                                            float alpha, float beta) {
    constexpr int E = 256 / G;
    __shared__ float part[G][E];
    const int el = threadIdx.x % E, g = threadIdx.x / E;
    const int q0 = (int)((int64_t)g * S / G), q1 = (int)((int64_t)(g + 1) * S / G);
    const int64_t plane = (int64_t)M * N;
    // The loop bound depends on the work-group only, so every work-item reaches
    // each barrier.
    for (int64_t base = (int64_t)blockIdx.x * E; base < plane; base += (int64_t)gridDim.x * E) {
        const int64_t e = base + el;
        float sum = 0.0f;
        if (e < plane) {
            const float *src = ws + e;
            int q = q0;
            for (; q + 16 <= q1; q += 16) {
                float v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = src[(q + u) * plane];
#pragma unroll
                for (int u = 0; u < 16; ++u) sum += v[u];
            }
            for (; q + 4 <= q1; q += 4) {
                float v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = src[(q + u) * plane];
#pragma unroll
                for (int u = 0; u < 4; ++u) sum += v[u];
            }
            for (; q < q1; ++q) sum += src[q * plane];
        }
        if constexpr (G > 1) {
            part[g][el] = sum;
            __syncthreads();
            if (g == 0) {
#pragma unroll
                for (int h = 1; h < G; ++h) sum += part[h][el];
            }
            __syncthreads();
        }
        if (g == 0 && e < plane) {
            const int64_t i = e / N, j = e - i * N;
            float *c = C + i * ldc + j;
            *c = epilogue(sum, alpha, beta, c);
        }
    }
}

// Plane groups per output element: the fewest (up to 16, at most S) that give
// 2048 work-groups, eight per CU.
static int splitk_reduce_groups(int64_t items, int slices) {
    int g = 1;
    while (g < 16 && 2 * g <= slices && (items * g + 255) / 256 < 2048) g *= 2;
    return g;
}

template <int G>
static hipError_t launch_reduce_g(const Problem &p, int slices, const float *ws, hipStream_t s) {
    constexpr int E = 256 / G;
    const int64_t items = (int64_t)p.M * p.N;
    int64_t blocks = (items + E - 1) / E;
    if (blocks > 16384) blocks = 16384;
    return launch(splitk_reduce_kernel<G>, dim3((unsigned)blocks), dim3(256), 0, s, p.M, p.N,
                  slices, ws, p.C, p.ldc, p.alpha, p.beta);
}

hipError_t launch_splitk_reduce(const Problem &p, int slices, const float *ws, hipStream_t s) {
    switch (splitk_reduce_groups((int64_t)p.M * p.N, slices)) {
        case 1: return launch_reduce_g<1>(p, slices, ws, s);
        case 2: return launch_reduce_g<2>(p, slices, ws, s);
        case 4: return launch_reduce_g<4>(p, slices, ws, s);
        case 8: return launch_reduce_g<8>(p, slices, ws, s);
        default: return launch_reduce_g<16>(p, slices, ws, s);
    }
}

// Element strides of op(A) (rows i, k) and op(B) (k, columns j).
struct Strides {
    int64_t ai, ak, bk, bj;
};

static Strides strides(const Problem &p) {
    return {p.ta ? 1 : p.lda, p.ta ? p.lda : 1, p.tb ? 1 : p.ldb, p.tb ? p.ldb : 1};
}

// ---------------------------------------------------------------------------
// Rung 0: one work-item per element of C, the sum over k read directly from
// global memory (page "CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结", §五;
// page "CUDA算子优化(4)：矩阵乘法", section "版本V1朴素矩阵乘法").
// A 64 x 4 work-group puts one wave on 64 consecutive columns of one row, so the
// reads of B and the store of C are contiguous across the wave and A[i][k] is a
// single address per wave.
constexpr int NAIVE_X = 64, NAIVE_Y = 4;

__global__ __launch_bounds__(NAIVE_X *NAIVE_Y) void naive_kernel(
    int M, int N, int K, const float *__restrict__ A, const float *__restrict__ B, Strides st,
    float *__restrict__ C, int64_t ldc, float alpha, float beta, int tiles_n) {
    int row, col;
    element_of(blockIdx.x, tiles_n, NAIVE_Y, NAIVE_X, threadIdx.x, threadIdx.y, &row, &col);
    if (row >= M || col >= N) return;
    const float *a = A + (int64_t)row * st.ai;
    const float *b = B + (int64_t)col * st.bj;
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum = fmaf(a[(int64_t)k * st.ak], b[(int64_t)k * st.bk], sum);
    float *c = C + (int64_t)row * ldc + col;
    *c = epilogue(sum, alpha, beta, c);
}

hipError_t launch_naive(const Problem &p, hipStream_t s) {
    const int64_t tiles_n = (p.N + NAIVE_X - 1) / NAIVE_X;
    const int64_t tiles_m = (p.M + NAIVE_Y - 1) / NAIVE_Y;
    if (tiles_n * tiles_m > INT32_MAX) return hipErrorInvalidValue;
    return launch(naive_kernel, dim3((unsigned)(tiles_n * tiles_m)), dim3(NAIVE_X, NAIVE_Y), 0, s,
                  p.M, p.N, p.K, p.A, p.B, strides(p), p.C, p.ldc, p.alpha, p.beta, (int)tiles_n);
}

// ---------------------------------------------------------------------------
// Rung 1: 16 x 16 output tile per work-group, A and B staged through LDS one
// 16 x 16 tile at a time (page "CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结",
// §六; page "【infra之路】Tiled Matrix Multiplication详解").  Partial tiles at the
// M, N and K edges are filled with zeros (§六, handling of sizes that are not a
// multiple of the tile), and there are two barriers per step: after the tile is
// written (before it is read) and after it is read (before it is overwritten).
// Rows are padded to 17 floats (§八, bank-conflict padding) so that the
// column-wise reads of the B tile fall in distinct banks.
constexpr int TILE = 16;

__global__ __launch_bounds__(TILE *TILE) void lds_tiled_kernel(
    int M, int N, int K, const float *__restrict__ A, const float *__restrict__ B, Strides st,
    float *__restrict__ C, int64_t ldc, float alpha, float beta, int tiles_n) {
    __shared__ float As[TILE][TILE + 1];
    __shared__ float Bs[TILE][TILE + 1];
    const int tx = threadIdx.x, ty = threadIdx.y;
    int row, col;
    element_of(blockIdx.x, tiles_n, TILE, TILE, tx, ty, &row, &col);
    float sum = 0.0f;
    for (int k0 = 0; k0 < K; k0 += TILE) {
        const int ka = k0 + tx, kb = k0 + ty;
        As[ty][tx] = (row < M && ka < K) ? A[(int64_t)row * st.ai + (int64_t)ka * st.ak] : 0.0f;
        Bs[ty][tx] = (kb < K && col < N) ? B[(int64_t)kb * st.bk + (int64_t)col * st.bj] : 0.0f;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TILE; ++k) sum = fmaf(As[ty][k], Bs[k][tx], sum);
        __syncthreads();
    }
    if (row < M && col < N) {
        float *c = C + (int64_t)row * ldc + col;
        *c = epilogue(sum, alpha, beta, c);
    }
}

hipError_t launch_lds_tiled(const Problem &p, hipStream_t s) {
    const int64_t tiles_n = (p.N + TILE - 1) / TILE;
    const int64_t tiles_m = (p.M + TILE - 1) / TILE;
    if (tiles_n * tiles_m > INT32_MAX) return hipErrorInvalidValue;
    return launch(lds_tiled_kernel, dim3((unsigned)(tiles_n * tiles_m)), dim3(TILE, TILE), 0, s,
                  p.M, p.N, p.K, p.A, p.B, strides(p), p.C, p.ldc, p.alpha, p.beta,
                  (int)tiles_n);
}

}  // namespace sgemm
