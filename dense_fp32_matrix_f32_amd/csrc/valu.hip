// valu.hip -- register-blocked vector-ALU rung of the ladder.
//
// The tiled scheme of the pages (page "CUDA算子优化(4)：矩阵乘法", section
// "版本V1共享内存分块"; page "GPU programming with C++ and CUDA", chapter 7,
// shared-memory tiles with unrolled inner loops and fused multiply-adds) with the
// per-thread work raised from one output to an 8 x 8 block:
//   * 128 x 128 block of C per 256-work-item work-group, 8-wide k windows;
//   * two LDS stages, next window loaded into registers one window ahead;
//   * A is stored k-major in LDS so that each work-item reads its 8 rows of A
//     and 8 columns of B for one k as four 16-byte LDS reads, then issues 64
//     v_fma_f32 (fp32 fused multiply-add, single rounding).
// A work-item's rows are ty*4 + {0..3} and 64 + ty*4 + {0..3} (same split for
// columns), so the 16 work-items that share an LDS row read 16 distinct 16-byte
// slots.  Edge handling is the one of the matrix-core rung: clamped row/column
// reads for outputs that are never stored, zero-filled final k window.
#include "internal.h"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 load16_valu(const float *p) {
    f32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

constexpr int VB = 128, VK = 8, VT = 256;
constexpr int VPITCH = VB + 4;

__global__ __launch_bounds__(VT) void valu_kernel(int M, int N, int K,
                                                  const float *__restrict__ A, int64_t lda,
                                                  const float *__restrict__ B, int64_t ldb,
                                                  float *__restrict__ C, int64_t ldc,
                                                  float alpha, float beta, int tiles_m,
                                                  int tiles_n) {
    __shared__ __attribute__((aligned(16))) float As[2][VK][VPITCH];
    __shared__ __attribute__((aligned(16))) float Bs[2][VK][VPITCH];

    int tm, tn;
    tile_order(blockIdx.x, tiles_m, tiles_n, 8, &tm, &tn);
    const int m0 = tm * VB, n0 = tn * VB;
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;

    // A window: 128 rows x 8 k = 256 vectors of 4 k; row tid/2, k quarter tid%2.
    const int a_r = tid >> 1, a_q = (tid & 1) * 4;
    const float *a_src = A + (int64_t)min(m0 + a_r, M - 1) * lda + a_q;
    // B window: 8 k x 128 columns = 256 vectors of 4 columns; k row tid/32.
    const int b_r = tid >> 5, b_c = (tid & 31) * 4;
    const int b_n = n0 + b_c;
    const float *b_src = B + (int64_t)b_r * ldb;

    f32x4 ra, rb;
    auto fetch = [&](int k0) {
        const bool tail = k0 + VK > K;
        if (!tail) {
            ra = load16_valu(a_src + k0);
        } else {
            const int kv = K - (k0 + a_q);
            const float *p = a_src + k0;
            ra.x = kv > 0 ? p[0] : 0.0f;
            ra.y = kv > 1 ? p[1] : 0.0f;
            ra.z = kv > 2 ? p[2] : 0.0f;
            ra.w = kv > 3 ? p[3] : 0.0f;
        }
        if (k0 + b_r < K) {
            const float *row = b_src + (int64_t)k0 * ldb;
            if (b_n + 3 < N) {
                rb = load16_valu(row + b_n);
            } else {
                rb.x = row[min(b_n + 0, N - 1)];
                rb.y = row[min(b_n + 1, N - 1)];
                rb.z = row[min(b_n + 2, N - 1)];
                rb.w = row[min(b_n + 3, N - 1)];
            }
        } else {
            rb = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    auto stash = [&](int st) {
        As[st][a_q + 0][a_r] = ra.x;
        As[st][a_q + 1][a_r] = ra.y;
        As[st][a_q + 2][a_r] = ra.z;
        As[st][a_q + 3][a_r] = ra.w;
        *(f32x4 *)&Bs[st][b_r][b_c] = rb;
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    const int windows = (K + VK - 1) / VK;
    fetch(0);
    stash(0);
    __syncthreads();
    if (windows > 1) fetch(VK);

    for (int w = 0; w < windows; ++w) {
        const int st = w & 1;
#pragma unroll
        for (int k = 0; k < VK; ++k) {
            const f32x4 a0 = *(const f32x4 *)&As[st][k][ty * 4];
            const f32x4 a1 = *(const f32x4 *)&As[st][k][64 + ty * 4];
            const f32x4 b0 = *(const f32x4 *)&Bs[st][k][tx * 4];
            const f32x4 b1 = *(const f32x4 *)&Bs[st][k][64 + tx * 4];
            const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        if (w + 1 < windows) {
            stash(st ^ 1);
            if (w + 2 < windows) fetch((w + 2) * VK);
        }
        __syncthreads();
    }

    const bool full = (m0 + VB <= M) && (n0 + VB <= N);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + i - 4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = n0 + h * 64 + tx * 4;
            float *dst = C + (int64_t)row * ldc + col;
            if (full) {
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[e] = epilogue(acc[i][h * 4 + e], alpha, beta, dst + e);
            } else if (row < M) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < N) dst[e] = epilogue(acc[i][h * 4 + e], alpha, beta, dst + e);
            }
        }
    }
}

hipError_t launch_valu_regblock(const Problem &p, hipStream_t s) {
    const int64_t tiles_m = (p.M + VB - 1) / VB, tiles_n = (p.N + VB - 1) / VB;
    if (tiles_m * tiles_n > INT32_MAX) return hipErrorInvalidValue;
    return launch(valu_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(VT), 0, s, p.M, p.N, p.K,
                  p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.alpha, p.beta, (int)tiles_m,
                  (int)tiles_n);
}

}  // namespace sgemm
