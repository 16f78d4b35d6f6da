// skinny.hip -- products with very few rows (M <= 8), e.g. a 1 x K row times K x N.
//
// With M = 1 the intensity formula of the page "CUDA算子优化(4)：矩阵乘法" (section
// "计算强度", I = MNK / (2(MK + KN + MN))) gives about 0.5 flop per byte, far below
// the chip's ridge point: the product is bound by reading B once from HBM.  The
// kernel therefore streams B exactly once with 16-byte loads, keeps up to 8 rows
// of A in flight per element of B, and splits K across the work-items of a
// work-group, followed by a reduction over the slots in a fixed order (across
// the lanes of each wave, then the waves in LDS), so results are reproducible and
// no atomics are needed.  With x contiguous along k, slot s takes runs of four
// consecutive k (4s .. 4s+3, then 4s + 4S .. 4s + 4S + 3, ...), so each run of x
// is one 16-byte load; with x strided along k it takes k = s, s + S, s + 2S, ...  Each work-group owns a strip of 4*LPR columns; with 16 columns (64
// bytes of a row) two work-groups share every 128-byte line, so strips are
// assigned XCD by XCD: neighbouring strips run on the same XCD and a line comes
// through its L2 once, not once per XCD.
//
// In general terms the kernel forms out[m][n] = alpha * sum_k x[m][k] * Y[k][n]
// + beta * out[m][n] for at most 8 rows m, with Y row-major (streamed) and x and
// out given by element strides, which covers every storage order: op(A) * B for
// few rows of C when B is not transposed, and (op(A) * op(B))^T = op(B)^T *
// A^T for few columns of C when A is transposed (Y is then the stored A).
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
// there are S = THREADS/LPR k slots.  MR is the number of rows of x handled.
// x[m][k] = A[m*xm + k*xk] (XK1: xk == 1), Y[k][n] = B[k*ldb + n], out[m][n] =
// C[m*cm + n*cn].
template <int MR, int LPR, int THREADS, bool XK1>
__global__ __launch_bounds__(THREADS) void skinny_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t xm, int64_t xk,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t cm, int64_t cn,
    float alpha, float beta) {
    constexpr int CW = 4 * LPR;        // columns per work-group
    constexpr int S = THREADS / LPR;   // k slots (a power of two)
    constexpr int OUT = MR * CW;       // outputs per work-group
    constexpr int U = MR <= 2 ? 16 : 8;  // k values per batch (loads in flight) per work-item
    static_assert((S & (S - 1)) == 0, "slot count is a power of two");
    static_assert(64 % LPR == 0, "whole slots in every wave");
    constexpr int WAVES = THREADS / 64;
    // partial sums: one row per wave (XK1) or per k slot, padded against bank conflicts
    __shared__ float red[XK1 ? WAVES : S][XK1 ? OUT : OUT + 1];

    const int tid = threadIdx.x;
    const int q = tid % LPR, slot = tid / LPR;
    const int n0 = xcd_remap(blockIdx.x, gridDim.x) * CW;
    const int n = n0 + 4 * q;
    const bool vec = n + 3 < N;

    const float *arow[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) arow[m] = A + (int64_t)min(m, M - 1) * xm;
    auto xat = [&](int m, int k) -> float {
        if constexpr (XK1) {
            return arow[m][k];
        } else {
            return arow[m][(int64_t)k * xk];
        }
    };

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
        if constexpr (XK1) {
            // One run of four consecutive k per step: four loads of B and one
            // 16-byte load per row of x in flight.  Against 16 single k per batch
            // (rows slot + u*S), back-to-back launches on the same box, B streamed
            // from HBM: 1 x 4096 x 4096 18.5 -> 17.6-17.8 us, 2 rows 18.6 -> 18.4,
            // 8 rows 22.4 -> 21.4, 1 x 8192 x 8192 68.3 -> 64.6; B resident: 1 x
            // 4096 x 4096 13.5 -> 13.0 us, 8 rows 15.3 -> 16.1.  More runs per
            // step, or pairs, were no faster, and some were twice as slow.
            int k = 4 * slot;
            for (; k + 3 < K; k += 4 * S) {
                f32x4 b[4];
                f32x4 a[MR];
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = load_b(k + j);
#pragma unroll
                for (int m = 0; m < MR; ++m) a[m] = load16_skinny(arow[m] + k);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float av[MR];
#pragma unroll
                    for (int m = 0; m < MR; ++m) av[m] = a[m][j];
                    fma4(av, b[j]);
                }
            }
            // the last run of a slot, cut by K
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (k + j < K) {
                    const f32x4 bv = load_b(k + j);
                    float av[MR];
#pragma unroll
                    for (int m = 0; m < MR; ++m) av[m] = arow[m][k + j];
                    fma4(av, bv);
                }
            return;
        }
        int k = slot;
        for (; k + (U - 1) * S < K; k += U * S) {
            f32x4 b[U];
            float a[U][MR];
#pragma unroll
            for (int u = 0; u < U; ++u) b[u] = load_b(k + u * S);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int m = 0; m < MR; ++m) a[u][m] = xat(m, k + u * S);
#pragma unroll
            for (int u = 0; u < U; ++u) fma4(a[u], b[u]);
        }
        for (; k < K; k += S) {
            const f32x4 b = load_b(k);
            float a[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) a[m] = xat(m, k);
            fma4(a, b);
        }
    };
    if (vec) {
        pass(std::true_type{});
    } else {
        pass(std::false_type{});
    }

    // The k slots, in a fixed order.  x contiguous along k: a butterfly across
    // the lanes of each wave (the slot bits of the lane index), then the waves'
    // sums added in wave order (one barrier).  x strided along k: a pairwise tree
    // over the slots in LDS (slot s absorbs slot s + stride); the butterfly
    // measured 1.7 times slower there at 8 x 4096 x 4096, whose loop already runs
    // out of registers.
    if constexpr (XK1) {
#pragma unroll
        for (int d = LPR; d < 64; d <<= 1)
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[m][e] += __shfl_xor(acc[m][e], d, 64);
        const int lane = tid & 63, wave = tid >> 6;
        if (lane < LPR) {
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[wave][m * CW + 4 * lane + e] = acc[m][e];
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[slot][m * CW + 4 * q + e] = acc[m][e];
        __syncthreads();
#pragma unroll
        for (int stride = S / 2; stride > 0; stride >>= 1) {
            for (int e = tid; e < stride * OUT; e += THREADS) {
                const int sl = e / OUT, o = e - sl * OUT;
                red[sl][o] += red[sl + stride][o];
            }
            __syncthreads();
        }
    }
    for (int o = tid; o < OUT; o += THREADS) {
        const int m = o / CW, c = o % CW;
        if (m < M && n0 + c < N) {
            float v = red[0][o];
            if constexpr (XK1) {
#pragma unroll
                for (int w = 1; w < WAVES; ++w) v += red[w][o];
            }
            float *dst = C + (int64_t)m * cm + (int64_t)(n0 + c) * cn;
            *dst = epilogue(v, alpha, beta, dst);
        }
    }
}

// One streaming product as above: x (rows x K, strides xm, xk), Y (K x cols,
// row stride ldy), out (rows x cols, strides cm, cn).
struct RowStream {
    int rows, cols, K;
    const float *x;
    int64_t xm, xk;
    const float *Y;
    int64_t ldy;
    float *out;
    int64_t cm, cn;
    float alpha, beta;
};

template <int MR, int THREADS, bool XK1>
static hipError_t launch_rows(const RowStream &q, hipStream_t s) {
    // Wide segments give longer contiguous row reads; narrow ones give more
    // work-groups.  Keep at least 256 work-groups (one per CU) when N allows.
    if (q.cols >= 64 * 256) {
        const int64_t groups = (q.cols + 63) / 64;
        return launch(skinny_kernel<MR, 16, THREADS, XK1>, dim3((unsigned)groups), dim3(THREADS),
                      0, s, q.rows, q.cols, q.K, q.x, q.xm, q.xk, q.Y, q.ldy, q.out, q.cm, q.cn,
                      q.alpha, q.beta);
    }
    const int64_t groups = (q.cols + 15) / 16;
    return launch(skinny_kernel<MR, 4, THREADS, XK1>, dim3((unsigned)groups), dim3(THREADS), 0, s,
                  q.rows, q.cols, q.K, q.x, q.xm, q.xk, q.Y, q.ldy, q.out, q.cm, q.cn, q.alpha,
                  q.beta);
}

template <int MR>
static hipError_t launch_rows_k1(const RowStream &q, hipStream_t s) {
    // x contiguous along k (runs of four k per slot): 512 work-items while the
    // strips give at most one work-group per CU, else 256 (measured on 1 to 8
    // rows of 1024 to 16384 columns, B resident and streamed from HBM).
    const int64_t groups = q.cols >= 64 * 256 ? (q.cols + 63) / 64 : (q.cols + 15) / 16;
    if (groups <= compute_units()) return launch_rows<MR, 512, true>(q, s);
    return launch_rows<MR, 256, true>(q, s);
}

template <bool XK1>
static hipError_t launch_rows_of(const RowStream &q, hipStream_t s) {
    if constexpr (XK1) {
        if (q.rows == 1) return launch_rows_k1<1>(q, s);
        if (q.rows == 2) return launch_rows_k1<2>(q, s);
        if (q.rows <= 4) return launch_rows_k1<4>(q, s);
        return launch_rows_k1<8>(q, s);
    } else {
        // Group sizes measured on 1..8 x 4096 x 4096 with B resident in the
        // Infinity Cache and streamed from HBM.
        if (q.rows == 1) return launch_rows<1, 256, false>(q, s);
        if (q.rows == 2) return launch_rows<2, 512, false>(q, s);
        if (q.rows <= 4) return launch_rows<4, 512, false>(q, s);
        return launch_rows<8, 256, false>(q, s);
    }
}

static hipError_t launch_row_stream(const RowStream &p, hipStream_t s) {
    if ((int64_t)(p.cols + 15) / 16 > INT32_MAX) return hipErrorInvalidValue;
    // More than 8 rows: one pass per group of 8 rows.
    for (int r0 = 0; r0 < p.rows; r0 += SKINNY_MAX_ROWS) {
        RowStream q = p;
        q.rows = p.rows - r0 < SKINNY_MAX_ROWS ? p.rows - r0 : SKINNY_MAX_ROWS;
        q.x = p.x + (int64_t)r0 * p.xm;
        q.out = p.out + (int64_t)r0 * p.cm;
        const hipError_t e = q.xk == 1 ? launch_rows_of<true>(q, s) : launch_rows_of<false>(q, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Few rows of C with B not transposed: x = op(A), Y = B, out = C.
hipError_t launch_skinny_rows(const Problem &p, hipStream_t s) {
    const RowStream q{p.M, p.N, p.K, p.A, p.ta ? 1 : p.lda, p.ta ? p.lda : 1, p.B, p.ldb,
                      p.C, p.ldc, 1, p.alpha, p.beta};
    return launch_row_stream(q, s);
}

// Few columns of C with A transposed: C^T = op(B)^T * A^T, so x = op(B)^T
// (N x K), Y = the stored K x M array A, out = C^T.
hipError_t launch_skinny_cols_ta(const Problem &p, hipStream_t s) {
    const RowStream q{p.N, p.M, p.K, p.B, p.tb ? p.ldb : 1, p.tb ? 1 : p.ldb, p.A, p.lda,
                      p.C, 1, p.ldc, p.alpha, p.beta};
    return launch_row_stream(q, s);
}

}  // namespace sgemm
