// mfma.hip -- register-blocked fp32 matrix-core rung of the ladder.
//
// Same decomposition as the pages' tiled kernel (page "CUDA算子优化(4)：矩阵乘法",
// section "版本V1共享内存分块": each work-group owns a TILE_M x TILE_N block of C and
// slides a TILE_K window along k, staging the A and B windows in on-chip memory),
// re-sized for gfx950:
//   * a BM x BN block of C per work-group, BK-wide k windows, two LDS stages
//     (the next window is written while the current one is read, so one barrier
//     per window replaces the pages' two);
//   * global -> LDS copies as 16-byte loads, issued one window ahead into
//     registers so that their latency overlaps a whole window of math;
//   * each wave owns a WM x WN sub-block held as (WM/32) x (WN/32) accumulators
//     of v_mfma_f32_32x32x2f32 (full fp32 inputs, fp32 accumulation, 4096 flops
//     per instruction), which is where the per-element fused multiply-adds of
//     the pages' kernels go;
//   * work-group ids are re-ordered so that each XCD works on one compact region
//     of C (see tile_order in internal.h).
//
// The k order inside one MFMA is fixed by the hardware; across MFMAs a lane
// half h supplies k = k8 + 4h + s for the s-th of four instructions, so each
// lane fetches four consecutive k of A with one 16-byte LDS read.  A and B use
// the same assignment, so every product A[i][k]*B[k][j] is formed exactly once.
//
// Edges: rows of A beyond M and columns of B beyond N are read from the last
// valid row/column (they only feed outputs that are not stored); the last,
// partial k window is zero-filled on both operands (the pages' zero-fill of
// partial tiles), so no value outside the logical matrices enters a stored
// result and no load leaves the matrices' extents.
#include "internal.h"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16-byte load from a 4-byte aligned address (gfx950 global loads accept
// dword-aligned dwordx4 accesses).
__device__ __forceinline__ f32x4 load16(const float *p) {
    f32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

template <int BM_, int BN_, int BK_, int WM_, int WN_, int GROUP_M_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int THREADS = WAVES_M * WAVES_N * 64;
    static constexpr int TM = WM / 32, TN = WN / 32;   // 32x32 accumulators per wave
    static constexpr int PA = BK + 4;                  // A row pitch in LDS (floats)
    static constexpr int PB = BN + 8;                  // B row pitch in LDS (floats)
    static constexpr int A_STAGE = BM * PA, B_STAGE = BK * PB;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_BYTES = 2 * STAGE * 4;
    static constexpr int A_VECS = BM * BK / 4 / THREADS;  // 16-byte loads per thread
    static constexpr int B_VECS = BK * BN / 4 / THREADS;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "wave tiling");
    static_assert(BK % 8 == 0, "k window is a multiple of 8");
    static_assert(A_VECS * THREADS * 4 == BM * BK && B_VECS * THREADS * 4 == BK * BN,
                  "loads divide evenly");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class T>
__global__ __launch_bounds__(T::THREADS) void mfma_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda, const float *__restrict__ B,
    int64_t ldb, float *__restrict__ C, int64_t ldc, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) float lds[2 * T::STAGE];

    int tm, tn;
    tile_order(blockIdx.x, tiles_m, tiles_n, T::GROUP_M, &tm, &tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

    // ---- global-load assignment (fixed for the whole k loop) ----
    constexpr int AQ = T::BK / 4;  // 16-byte vectors per A row of the window
    constexpr int BQ = T::BN / 4;  // 16-byte vectors per B row of the window
    const float *a_src[T::A_VECS];
    int a_lds[T::A_VECS], a_k[T::A_VECS];
#pragma unroll
    for (int v = 0; v < T::A_VECS; ++v) {
        const int c = tid + v * T::THREADS;
        const int r = c / AQ, q = c % AQ;
        const int gr = min(m0 + r, M - 1);
        a_k[v] = q * 4;
        a_src[v] = A + (int64_t)gr * lda + q * 4;
        a_lds[v] = r * T::PA + q * 4;
    }
    const float *b_src[T::B_VECS];
    int b_lds[T::B_VECS], b_k[T::B_VECS], b_n[T::B_VECS];
#pragma unroll
    for (int v = 0; v < T::B_VECS; ++v) {
        const int c = tid + v * T::THREADS;
        const int r = c / BQ, q = c % BQ;
        b_k[v] = r;
        b_n[v] = n0 + q * 4;
        b_src[v] = B + (int64_t)r * ldb + n0 + q * 4;
        b_lds[v] = T::A_STAGE + r * T::PB + q * 4;
    }

    f32x4 ra[T::A_VECS], rb[T::B_VECS];

    // Loads of the k window starting at k0 into registers.
    auto fetch = [&](int k0) {
        if (k0 + T::BK <= K) {
#pragma unroll
            for (int v = 0; v < T::A_VECS; ++v) ra[v] = load16(a_src[v] + k0);
#pragma unroll
            for (int v = 0; v < T::B_VECS; ++v) {
                const float *p = b_src[v] + (int64_t)k0 * ldb;
                if (b_n[v] + 3 < N) {
                    rb[v] = load16(p);
                } else {
                    const int base = b_n[v];
                    const float *row = p - base;
                    rb[v].x = row[min(base + 0, N - 1)];
                    rb[v].y = row[min(base + 1, N - 1)];
                    rb[v].z = row[min(base + 2, N - 1)];
                    rb[v].w = row[min(base + 3, N - 1)];
                }
            }
        } else {
            // Last, partial window: zero every element with k >= K.
#pragma unroll
            for (int v = 0; v < T::A_VECS; ++v) {
                const int kv = K - (k0 + a_k[v]);
                const float *p = a_src[v] + k0;
                ra[v].x = kv > 0 ? p[0] : 0.0f;
                ra[v].y = kv > 1 ? p[1] : 0.0f;
                ra[v].z = kv > 2 ? p[2] : 0.0f;
                ra[v].w = kv > 3 ? p[3] : 0.0f;
            }
#pragma unroll
            for (int v = 0; v < T::B_VECS; ++v) {
                if (k0 + b_k[v] < K) {
                    const int base = b_n[v];
                    const float *row = b_src[v] + (int64_t)k0 * ldb - base;
                    rb[v].x = row[min(base + 0, N - 1)];
                    rb[v].y = row[min(base + 1, N - 1)];
                    rb[v].z = row[min(base + 2, N - 1)];
                    rb[v].w = row[min(base + 3, N - 1)];
                } else {
                    rb[v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
        }
    };
    auto stash = [&](int stage) {
        float *s = lds + stage * T::STAGE;
#pragma unroll
        for (int v = 0; v < T::A_VECS; ++v) *(f32x4 *)(s + a_lds[v]) = ra[v];
#pragma unroll
        for (int v = 0; v < T::B_VECS; ++v) *(f32x4 *)(s + b_lds[v]) = rb[v];
    };

    f32x16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = f32x16{};

    const int a_frag = (wm * T::WM + lr) * T::PA + 4 * lh;
    const int b_frag = T::A_STAGE + (4 * lh) * T::PB + wn * T::WN + lr;

    const int windows = (K + T::BK - 1) / T::BK;
    fetch(0);
    stash(0);
    __syncthreads();
    if (windows > 1) fetch(T::BK);

    for (int w = 0; w < windows; ++w) {
        const float *s = lds + (w & 1) * T::STAGE;
#pragma unroll
        for (int k8 = 0; k8 < T::BK; k8 += 8) {
            f32x4 af[T::TM];
            float bf[T::TN][4];
#pragma unroll
            for (int i = 0; i < T::TM; ++i) af[i] = *(const f32x4 *)(s + a_frag + i * 32 * T::PA + k8);
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) bf[j][q] = s[b_frag + (k8 + q) * T::PB + j * 32];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < T::TM; ++i)
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][q], bf[j][q],
                                                                          acc[i][j], 0, 0, 0);
        }
        if (w + 1 < windows) {
            stash((w + 1) & 1);
            if (w + 2 < windows) fetch((w + 2) * T::BK);
        }
        __syncthreads();
    }

    // ---- epilogue: accumulator r of block (i, j) holds row 8*(r/4) + 4*lh + r%4, column lr ----
    const bool full = (m0 + T::BM <= M) && (n0 + T::BN <= N);
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int col = n0 + wn * T::WN + j * 32 + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * T::WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (full || (row < M && col < N)) C[(int64_t)row * ldc + col] = acc[i][j][r];
            }
        }
    }
}

template <class T>
static hipError_t launch_tile(const Problem &p, hipStream_t s) {
    const int64_t tiles_m = (p.M + T::BM - 1) / T::BM;
    const int64_t tiles_n = (p.N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > INT32_MAX) return hipErrorInvalidValue;
    return launch(mfma_kernel<T>, dim3((unsigned)(tiles_m * tiles_n)), dim3(T::THREADS), 0, s,
                  p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, (int)tiles_m, (int)tiles_n);
}

using TileLarge = MfmaTile<128, 256, 16, 64, 128, 8>;
using TileMedium = MfmaTile<128, 128, 16, 64, 64, 8>;
using TileSmall = MfmaTile<64, 64, 16, 32, 32, 4>;

hipError_t launch_mfma(const Problem &p, hipStream_t s) {
    const int64_t big = (int64_t)((p.M + 127) / 128) * ((p.N + 255) / 256);
    const int64_t mid = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128);
    if (big >= 512) return launch_tile<TileLarge>(p, s);
    if (mid >= 256) return launch_tile<TileMedium>(p, s);
    return launch_tile<TileSmall>(p, s);
}

}  // namespace sgemm
