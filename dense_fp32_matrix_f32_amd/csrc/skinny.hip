// skinny.hip -- products with very few rows (M <= 8), e.g. a 1 x K row times K x N.
//
// With M = 1 the intensity formula of the page "CUDA算子优化(4)：矩阵乘法" (section
// "计算强度", I = MNK / (2(MK + KN + MN))) gives about 0.5 flop per byte, far below
// the chip's ridge point: the product is bound by reading B once from HBM.  The
// kernel therefore streams B exactly once with 16-byte loads, keeps up to 8 rows
// of A in flight per element of B, and splits K across the work-items of a
// work-group (k = slot, slot + S, slot + 2S, ...), followed by a fixed-order
// pairwise reduction in LDS, so results are reproducible and no atomics are
// needed.  Each work-group owns a strip of 4*LPR columns; with 16 columns (64
// bytes of a row) two work-groups share every 128-byte line, so strips are
// assigned XCD by XCD: neighbouring strips run on the same XCD and a line comes
// through its L2 once, not once per XCD.
#include <type_traits>

#include "internal.h"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SKINNY_MAX_ROWS = 8;

__device__ __forceinline__ f32x4 load16_skinny(const float *p) {
    f32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// THREADS work-items; LPR of them share one row segment of 4*LPR columns, so
// there are S = THREADS/LPR k slots.  MR is the number of rows of A handled.
template <int MR, int LPR, int THREADS>
__global__ __launch_bounds__(THREADS) void skinny_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda, const float *__restrict__ B,
    int64_t ldb, float *__restrict__ C, int64_t ldc, float alpha, float beta) {
    constexpr int CW = 4 * LPR;        // columns per work-group
    constexpr int S = THREADS / LPR;   // k slots (a power of two)
    constexpr int OUT = MR * CW;       // outputs per work-group
    constexpr int U = MR <= 2 ? 16 : 8;  // k values per batch (loads in flight) per work-item
    static_assert((S & (S - 1)) == 0, "slot count is a power of two");
    __shared__ float red[S][OUT + 1];

    const int tid = threadIdx.x;
    const int q = tid % LPR, slot = tid / LPR;
    const int n0 = xcd_remap(blockIdx.x, gridDim.x) * CW;
    const int n = n0 + 4 * q;
    const bool vec = n + 3 < N;

    const float *arow[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) arow[m] = A + (int64_t)min(m, M - 1) * lda;

    float acc[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m][0] = acc[m][1] = acc[m][2] = acc[m][3] = 0.0f;

    // One pass over this work-item's k values.  VEC: its four columns lie inside
    // B (every work-item but those at the right edge), read as one 16-byte load;
    // otherwise column indices are clamped to N - 1 (those outputs are not stored).
    // All loads of a batch of U k values are issued before any of them is used,
    // so U loads of B and U*MR values of A are in flight together.
    auto pass = [&](auto vec_tag) {
        constexpr bool VEC = decltype(vec_tag)::value;
        int cn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) cn[e] = min(n + e, N - 1);
        auto load_b = [&](int k) -> f32x4 {
            const float *row = B + (int64_t)k * ldb;
            if constexpr (VEC) {
                return load16_skinny(row + n);
            } else {
                f32x4 v;
                v.x = row[cn[0]];
                v.y = row[cn[1]];
                v.z = row[cn[2]];
                v.w = row[cn[3]];
                return v;
            }
        };
        auto fma4 = [&](const float (&a)[MR], const f32x4 &b) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                acc[m][0] = fmaf(a[m], b.x, acc[m][0]);
                acc[m][1] = fmaf(a[m], b.y, acc[m][1]);
                acc[m][2] = fmaf(a[m], b.z, acc[m][2]);
                acc[m][3] = fmaf(a[m], b.w, acc[m][3]);
            }
        };
        int k = slot;
        for (; k + (U - 1) * S < K; k += U * S) {
            f32x4 b[U];
            float a[U][MR];
#pragma unroll
            for (int u = 0; u < U; ++u) b[u] = load_b(k + u * S);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int m = 0; m < MR; ++m) a[u][m] = arow[m][k + u * S];
#pragma unroll
            for (int u = 0; u < U; ++u) fma4(a[u], b[u]);
        }
        for (; k < K; k += S) {
            const f32x4 b = load_b(k);
            float a[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) a[m] = arow[m][k];
            fma4(a, b);
        }
    };
    if (vec) {
        pass(std::true_type{});
    } else {
        pass(std::false_type{});
    }

#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[slot][m * CW + 4 * q + e] = acc[m][e];
    __syncthreads();

    // Fixed pairwise tree over the k slots: slot s absorbs slot s + stride.
#pragma unroll
    for (int stride = S / 2; stride > 0; stride >>= 1) {
        for (int e = tid; e < stride * OUT; e += THREADS) {
            const int sl = e / OUT, o = e - sl * OUT;
            red[sl][o] += red[sl + stride][o];
        }
        __syncthreads();
    }
    for (int o = tid; o < OUT; o += THREADS) {
        const int m = o / CW, c = o % CW;
        if (m < M && n0 + c < N) {
            float *dst = C + (int64_t)m * ldc + n0 + c;
            *dst = epilogue(red[0][o], alpha, beta, dst);
        }
    }
}

template <int MR, int THREADS>
static hipError_t launch_rows(const Problem &p, hipStream_t s) {
    // Wide segments give longer contiguous row reads; narrow ones give more
    // work-groups.  Keep at least 256 work-groups (one per CU) when N allows.
    if (p.N >= 64 * 256) {
        const int64_t groups = (p.N + 63) / 64;
        return launch(skinny_kernel<MR, 16, THREADS>, dim3((unsigned)groups), dim3(THREADS), 0, s,
                      p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.alpha, p.beta);
    }
    const int64_t groups = (p.N + 15) / 16;
    return launch(skinny_kernel<MR, 4, THREADS>, dim3((unsigned)groups), dim3(THREADS), 0, s, p.M,
                  p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.alpha, p.beta);
}

hipError_t launch_skinny(const Problem &p, hipStream_t s) {
    if ((int64_t)(p.N + 15) / 16 > INT32_MAX) return hipErrorInvalidValue;
    // More than 8 rows: one pass per group of 8 rows.
    for (int r0 = 0; r0 < p.M; r0 += SKINNY_MAX_ROWS) {
        Problem q = p;
        q.M = p.M - r0 < SKINNY_MAX_ROWS ? p.M - r0 : SKINNY_MAX_ROWS;
        q.A = p.A + (int64_t)r0 * p.lda;
        q.C = p.C + (int64_t)r0 * p.ldc;
        hipError_t e;
        // Group sizes measured on 1..8 x 4096 x 4096 with B resident in the
        // Infinity Cache and streamed from HBM.
        if (q.M == 1) e = launch_rows<1, 256>(q, s);
        else if (q.M == 2) e = launch_rows<2, 512>(q, s);
        else if (q.M <= 4) e = launch_rows<4, 512>(q, s);
        else e = launch_rows<8, 256>(q, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sgemm
