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
//
// In general terms the kernel forms out[i][j] = alpha * sum_k X[i][k] * y[k][j]
// + beta * out[i][j] for at most 8 columns j, with X's rows contiguous along k
// (streamed) and y and out given by element strides, which covers every storage
// order: A * op(B) for few columns of C when A is not transposed, and
// (op(A) * op(B))^T = B^T * op(A)^T for few rows of C when B is transposed (X is
// then the stored N x K array B: a row vector times a transposed weight matrix).
#include "internal.h"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SKINNY_N_MAX_COLS = 8;
// Values of k per LDS chunk of y (YM 5): 1024 for one column, 2048 for more
// (sweeps of 512, 1024 and 2048 over 1 and 2 columns, 1023 to 8192 k).
template <int NR>
constexpr int skinny_n_chunk() {
    return NR == 1 ? 1024 : 2048;
}

__device__ __forceinline__ f32x4 load16_n(const float *p) {
    f32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// NR columns handled (N <= NR), RW rows per wave, 4 waves per work-group.
// X[i][k] = A[i*lda + k], y[k][j] = B[k*yk + j*yj], out[i][j] = C[i*ci + j*cj].
// YM: how a lane reads its four k of y: 0 one value at a time, 1 whole rows of y
// as 16-byte loads (yj == 1 and N == NR >= 4), 2 four consecutive k of each
// column as one 16-byte load (yk == 1), 3 rows of y as NR values although N <
// NR (yj == 1, yk + N >= NR): the values past column N - 1 come from the next
// row or the row padding of y and only feed outputs that are not stored; the
// last four k rows, where that would read past the matrix, go value by value;
// 4 (NR == N == 2, y dense: yk == 2, yj == 1) a lane's four rows are eight
// consecutive floats, read as two 16-byte loads; 5 (y's rows far apart, e.g. a
// few columns of a wide B) chunks of skinny_n_chunk() values of k (all columns)
// are gathered into LDS once per work-group, zero past K, and each lane
// reads its four k of a column there as one 16-byte read.  Read value by value,
// every wave touches one cache line per value of y (64 lines per load
// instruction against 8 for its row of X); the gather does that once per
// work-group.  The k order of every lane is the same in all modes, so the
// results are too.  U (y read from memory): steps of 256 k whose loads are all
// issued before any of them is used.
template <int NR, int RW, int YM, int U = 1>
__global__ __launch_bounds__(256) void skinny_n_kernel(int M, int N, int K,
                                                       const float *__restrict__ A, int64_t lda,
                                                       const float *__restrict__ B, int64_t yk,
                                                       int64_t yj, float *__restrict__ C,
                                                       int64_t ci, int64_t cj, float alpha,
                                                       float beta) {
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

    // The four k from k on (k + 3 < K) of the lane's rows of X and of y.
    auto load_full = [&](int k, f32x4 (&a)[RW], float (&b)[4][NR]) {
#pragma unroll
            for (int r = 0; r < RW; ++r) a[r] = load16_n(arow[r] + k);
            if constexpr (YM == 1 || YM == 3) {
                if (YM == 1 || k + 4 < K) {
                    // Whole rows of y: NR/4 16-byte loads per k.
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int j4 = 0; j4 < NR / 4; ++j4) {
                            const f32x4 v = load16_n(B + (int64_t)(k + e) * yk + 4 * j4);
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
                            b[e][j] = B[(int64_t)(k + e) * yk + min(j, N - 1)];
                }
            } else if constexpr (YM == 4) {
                const f32x4 v0 = load16_n(B + (int64_t)k * 2);
                const f32x4 v1 = load16_n(B + (int64_t)k * 2 + 4);
                b[0][0] = v0.x;
                b[0][1] = v0.y;
                b[1][0] = v0.z;
                b[1][1] = v0.w;
                b[2][0] = v1.x;
                b[2][1] = v1.y;
                b[3][0] = v1.z;
                b[3][1] = v1.w;
            } else if constexpr (YM == 2) {
                // Columns of y contiguous along k: one 16-byte load per column.
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    const f32x4 v = load16_n(B + (int64_t)min(j, N - 1) * yj + k);
                    b[0][j] = v.x;
                    b[1][j] = v.y;
                    b[2][j] = v.z;
                    b[3][j] = v.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int j = 0; j < NR; ++j)
                        b[e][j] = B[(int64_t)(k + e) * yk + (int64_t)min(j, N - 1) * yj];
            }
    };
    auto fma_step = [&](const f32x4 (&a)[RW], const float (&b)[4][NR]) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                acc[r][j] = fmaf(a[r].x, b[0][j], acc[r][j]);
                acc[r][j] = fmaf(a[r].y, b[1][j], acc[r][j]);
                acc[r][j] = fmaf(a[r].z, b[2][j], acc[r][j]);
                acc[r][j] = fmaf(a[r].w, b[3][j], acc[r][j]);
            }
    };

    if constexpr (YM != 5) {
    int k = 4 * lane;
    if constexpr (U > 1) {
        // whole batches of U steps
        for (; k + 256 * (U - 1) + 3 < K; k += 256 * U) {
            f32x4 a[U][RW];
            float b[U][4][NR];
#pragma unroll
            for (int u = 0; u < U; ++u) load_full(k + 256 * u, a[u], b[u]);
#pragma unroll
            for (int u = 0; u < U; ++u) fma_step(a[u], b[u]);
        }
    }
    for (; k < K; k += 256) {
        f32x4 a[RW];
        float b[4][NR];
        if (k + 3 < K) {
            load_full(k, a, b);
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
                    b[e][j] = k + e < K ? B[(int64_t)(k + e) * yk + (int64_t)min(j, N - 1) * yj]
                                        : 0.0f;
        }
        fma_step(a, b);
    }
    } else {
        // Work-item t gathers the values (k, j) of the chunk with k * NR + j = t +
        // 256 i, so adjacent columns of one k come from adjacent work-items.  The
        // gather completes before the chunk is used: the loads of X queue behind
        // any load issued before them, and the gathered ones are slow.
        constexpr int KC = skinny_n_chunk<NR>();  // k per chunk
        constexpr int PER = NR * KC / 256;        // values gathered per work-item
        static_assert(KC % 256 == 0, "a chunk holds whole 256-wide steps of the lanes");
        __shared__ __attribute__((aligned(16))) float yl[NR * KC];
        for (int k0 = 0; k0 < K; k0 += KC) {
            if (k0 > 0) __syncthreads();  // the previous chunk has been read
            float g[PER];
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int u = threadIdx.x + 256 * i;
                const int k = k0 + u / NR, j = u % NR;
                g[i] = k < K ? B[(int64_t)k * yk + (int64_t)min(j, N - 1) * yj] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int u = threadIdx.x + 256 * i;
                yl[(u % NR) * KC + u / NR] = g[i];
            }
            __syncthreads();
            const int kend = min(K, k0 + KC);
            for (int k = k0 + 4 * lane; k < kend; k += 256) {
                f32x4 a[RW];
                if (k + 3 < K) {
#pragma unroll
                    for (int r = 0; r < RW; ++r) a[r] = load16_n(arow[r] + k);
                } else {
#pragma unroll
                    for (int r = 0; r < RW; ++r) {
                        a[r].x = arow[r][k];
                        a[r].y = k + 1 < K ? arow[r][k + 1] : 0.0f;
                        a[r].z = k + 2 < K ? arow[r][k + 2] : 0.0f;
                        a[r].w = k + 3 < K ? arow[r][k + 3] : 0.0f;
                    }
                }
                f32x4 b[NR];
#pragma unroll
                for (int j = 0; j < NR; ++j) b[j] = *(const f32x4 *)(yl + j * KC + (k - k0));
#pragma unroll
                for (int r = 0; r < RW; ++r)
#pragma unroll
                    for (int j = 0; j < NR; ++j) {
                        acc[r][j] = fmaf(a[r].x, b[j].x, acc[r][j]);
                        acc[r][j] = fmaf(a[r].y, b[j].y, acc[r][j]);
                        acc[r][j] = fmaf(a[r].z, b[j].z, acc[r][j]);
                        acc[r][j] = fmaf(a[r].w, b[j].w, acc[r][j]);
                    }
            }
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
                        float *dst = C + (int64_t)(row0 + r) * ci + (int64_t)j * cj;
                        *dst = epilogue(acc[r][j], alpha, beta, dst);
                    }
    }
}

// One streaming product as above: X (rows x K, row stride ldx), y (K x cols,
// strides yk, yj), out (rows x cols, strides ci, cj).
struct ColStream {
    int rows, cols, K;
    const float *X;
    int64_t ldx;
    const float *y;
    int64_t yk, yj;
    float *out;
    int64_t ci, cj;
    float alpha, beta;
};

template <int NR, int RW, int YM, int U>
static hipError_t launch_cols_u(const ColStream &q, hipStream_t s) {
    const int64_t groups = (q.rows + 4 * RW - 1) / (4 * RW);
    if (groups > INT32_MAX) return hipErrorInvalidValue;
    return launch(skinny_n_kernel<NR, RW, YM, U>, dim3((unsigned)groups), dim3(256), 0, s, q.rows,
                  q.cols, q.K, q.X, q.ldx, q.y, q.yk, q.yj, q.out, q.ci, q.cj, q.alpha, q.beta);
}

// Steps per batch.  With y read along k (YM 2) or two dense columns (YM 4), two
// rows per wave and at most four columns: eight steps of 256 k per batch when K
// >= 2048 (four with four columns), four when K is shorter, one step at a time
// otherwise.  Against one step at a time (back-to-back launches, the same box):
// 4096 x 1 x 4096 11.9 -> 11.4 us, 2048 x 1 x 16384 30.7 -> 25.0 us, a row times
// a transposed 4096 x 4096 matrix streamed from HBM 14.9 -> 13.9 us, 4096 x 2 x
// 4096 level.  With y gathered into LDS (YM 5) four steps per batch made the
// last column of 4095 x 4097 x 1023 slower (6.35 -> 6.84 us traced), and the
// modes that read whole rows of y lost as well; they take one step at a time.
template <int NR, int RW, int YM>
static hipError_t launch_cols(const ColStream &q, hipStream_t s) {
    constexpr bool BATCH = RW == 2 && (YM == 2 || YM == 4) && NR <= 4;
    if constexpr (BATCH) {
        constexpr int UMAX = NR == 4 ? 4 : 8;
        if (UMAX >= 8 && q.K >= 2048) return launch_cols_u<NR, RW, YM, (UMAX >= 8 ? 8 : 1)>(q, s);
        if (q.K > 768) return launch_cols_u<NR, RW, YM, 4>(q, s);  // four steps per lane
    }
    return launch_cols_u<NR, RW, YM, 1>(q, s);
}

// Rows per wave.  More rows re-use each value of y more often; fewer give more
// work-groups and fewer loads of y per load of X.  Measured on 2048 to 16384
// rows of 4096 k: two rows when y is read along k (YM 2) and for one column or
// four whole columns (1.3 to 1.7 times faster than eight rows at 4096 rows); in
// the other cases (y read value by value, or eight columns) the most rows that
// still give 256 work-groups (with y gathered into LDS, YM 5, one column kept
// two rows: four or eight were up to 2% slower at 4096 and 16384 rows).
template <int NR, int YM>
static hipError_t launch_cols_rw(const ColStream &q, hipStream_t s) {
    const bool two = YM == 2 || YM == 4 || NR == 1 || (NR == 4 && (YM == 1 || YM == 3));
    if (!two && (int64_t)q.rows >= 4 * 8 * 256) return launch_cols<NR, 8, YM>(q, s);
    if (!two && (int64_t)q.rows >= 4 * 4 * 256) return launch_cols<NR, 4, YM>(q, s);
    return launch_cols<NR, 2, YM>(q, s);
}

template <int NR>
static hipError_t launch_cols_of(const ColStream &q, hipStream_t s) {
    if constexpr (NR == 2) {
        if (q.cols == 2 && q.yj == 1 && q.yk == 2) return launch_cols_rw<NR, 4>(q, s);
    }
    if constexpr (NR >= 4) {
        if (q.cols == NR && q.yj == 1) return launch_cols_rw<NR, 1>(q, s);
        if (q.yj == 1 && q.yk != 1 && q.yk + q.cols >= NR) return launch_cols_rw<NR, 3>(q, s);
    }
    if (q.yk == 1) return launch_cols_rw<NR, 2>(q, s);
    // y's rows at least a cache line apart: gathered into LDS (with four or eight
    // columns one of y's strides is 1, which the cases above take)
    if constexpr (NR <= 2) {
        if (q.K >= 256 && q.yk >= 32) return launch_cols_rw<NR, 5>(q, s);
    }
    return launch_cols_rw<NR, 0>(q, s);
}

static hipError_t launch_col_stream(const ColStream &p, hipStream_t s) {
    // More than 8 columns: one pass per group of 8 columns.
    for (int c0 = 0; c0 < p.cols; c0 += SKINNY_N_MAX_COLS) {
        ColStream q = p;
        q.cols = p.cols - c0 < SKINNY_N_MAX_COLS ? p.cols - c0 : SKINNY_N_MAX_COLS;
        q.y = p.y + (int64_t)c0 * p.yj;
        q.out = p.out + (int64_t)c0 * p.cj;
        hipError_t e;
        if (q.cols == 1) e = launch_cols_of<1>(q, s);
        else if (q.cols == 2) e = launch_cols_of<2>(q, s);
        else if (q.cols <= 4) e = launch_cols_of<4>(q, s);
        else e = launch_cols_of<8>(q, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Few columns of C with A not transposed: X = A, y = op(B), out = C.
hipError_t launch_skinny_cols(const Problem &p, hipStream_t s) {
    const ColStream q{p.M, p.N, p.K, p.A, p.lda, p.B, p.tb ? 1 : p.ldb, p.tb ? p.ldb : 1,
                      p.C, p.ldc, 1, p.alpha, p.beta};
    return launch_col_stream(q, s);
}

// Few rows of C with B transposed: C^T = B^T * op(A)^T, so X = the stored N x K
// array B, y = op(A)^T (K x M), out = C^T.
hipError_t launch_skinny_rows_tb(const Problem &p, hipStream_t s) {
    const ColStream q{p.N, p.M, p.K, p.B, p.ldb, p.A, p.ta ? p.lda : 1, p.ta ? 1 : p.lda,
                      p.C, 1, p.ldc, p.alpha, p.beta};
    return launch_col_stream(q, s);
}

}  // namespace sgemm
