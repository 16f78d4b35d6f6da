// split.hip -- the fp32 product on the bf16 matrix cores: each operand value is
// split into three bf16 parts and six of the nine part products are summed.
//
// The pages' last optimisation step is the matrix units of their GPU ("Tensor
// Core", page "CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结", the summary and
// outlook sections).  gfx950 has no reduced-precision fp32 matrix format, but its
// bf16 matrix cores do sixteen times the fp32 matrix-core work per cycle.  A
// float x is the exact sum x0 + x1 + x2 of three bf16 values (x0 = bf16(x),
// x1 = bf16(x - x0), x2 = bf16(x - x0 - x1); each residual is exact in fp32 and
// each part keeps the next 8 significant bits), and a bf16 x bf16 product is
// exact in fp32.  So
//     a*b = sum over p, q of ap*bq,
// and the products with p + q <= 2 (six of nine: a0b0, a0b1, a1b0, a0b2, a1b1,
// a2b0) carry everything above about 2^-24 of |a*b|; the three dropped ones are
// below it.  The sum is accumulated in fp32 by the matrix cores, smallest terms
// first, so the result has the error of an fp32 product: all-ones, identity and
// small-integer products stay exact.  Values whose bf16 rounding overflows (|x|
// above about 3.39e38) become infinite, and an infinite input makes its row or
// column of C NaN rather than +-Inf (its residual parts are not numbers).
//
// Layout of the work is that of the fp32 rung (mfma_kernel.h): a 256 x 128 block
// of C per work-group, four waves of 128 x 64, k windows of 16 in a three-stage
// LDS ring with one barrier per window and the next window's fragments read
// during the current one's MFMAs.  Global loads run two windows ahead into
// registers; the split into parts happens when a window goes from registers to
// LDS, so each value is split once per work-group.  Both operands are kept in
// LDS with k contiguous (B is gathered column by column from global memory), as
// rows of 16 bf16 per part whose two 16-byte halves swap places on every other
// group of 8 rows, which keeps the fragment reads free of bank conflicts.
// v_mfma_f32_32x32x16_bf16: lane l supplies row (column) l % 32 and eight
// consecutive k starting at 8*(l / 32), the same k for A and B.
#include "mfma_kernel.h"

namespace sgemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

namespace split {

constexpr int BM = 256, BN = 128, BK = 16;
constexpr int WM = 128, WN = 64, TM = WM / 32, TN = WN / 32;
constexpr int WAVES_N = BN / WN;
constexpr int THREADS = (BM / WM) * WAVES_N * 64;
constexpr int STAGES = 3;
constexpr int PARTS = 3;
constexpr int GROUP_M = 8;
// bf16 elements of one part of one operand window, and of one LDS stage
constexpr int A_PART = BM * BK, B_PART = BN * BK;
constexpr int STAGE = PARTS * (A_PART + B_PART);
// global -> register work per thread and window: A as runs of 8 k of one row,
// B as runs of 8 k of one column
constexpr int A_RUNS = BM * BK / 8 / THREADS;
constexpr int B_RUNS = BN * BK / 8 / THREADS;
static_assert(A_RUNS * THREADS * 8 == BM * BK && B_RUNS * THREADS * 8 == BN * BK, "whole runs");
static_assert(STAGES * STAGE * 2 <= 160 * 1024, "LDS budget");

// Element offset (bf16 units) of the 8-wide k half `h` of row `row` in a part.
__device__ __forceinline__ int slot(int row, int h) { return row * BK + 8 * (h ^ ((row >> 3) & 1)); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// bf16 pair (round to nearest even, v_cvt_pk_bf16_f32) as one 32-bit word.
__device__ __forceinline__ unsigned to_bf16x2(float x, float y) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x, y}, bf16x2));
}

// The three bf16 parts of eight floats (see the file comment), two at a time:
// the value of a part is read back from its bits, so each pair needs one
// conversion per part.  An infinite input leaves NaN residuals.
__device__ __forceinline__ void split3(const f32x8 &x, bf16x8 &p0, bf16x8 &p1, bf16x8 &p2) {
    u32x4 w0, w1, w2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a = x[2 * e], b = x[2 * e + 1];
        const unsigned u0 = to_bf16x2(a, b);
        const float ra = a - __builtin_bit_cast(float, u0 << 16);
        const float rb = b - __builtin_bit_cast(float, u0 & 0xffff0000u);
        const unsigned u1 = to_bf16x2(ra, rb);
        const float sa = ra - __builtin_bit_cast(float, u1 << 16);
        const float sb = rb - __builtin_bit_cast(float, u1 & 0xffff0000u);
        w0[e] = u0;
        w1[e] = u1;
        w2[e] = to_bf16x2(sa, sb);
    }
    p0 = __builtin_bit_cast(bf16x8, w0);
    p1 = __builtin_bit_cast(bf16x8, w1);
    p2 = __builtin_bit_cast(bf16x8, w2);
}

// The six part products (p, q), smallest first.
constexpr int PP[6][2] = {{2, 0}, {1, 1}, {0, 2}, {1, 0}, {0, 1}, {0, 0}};

struct Args {
    int M, N, K;
    const float *__restrict__ A;
    int64_t lda;
    const float *__restrict__ B;
    int64_t ldb;
    float *__restrict__ C;
    int64_t ldc;
    float alpha, beta;
};

__global__ __launch_bounds__(THREADS, 1) void split_kernel(Args g, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) __bf16 lds[STAGES * STAGE];
    const int M = g.M, N = g.N, K = g.K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    tile_order(blockIdx.x, tiles_m, tiles_n, GROUP_M, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- global -> register assignment ----
    const float *a_src[A_RUNS];
    int a_row[A_RUNS], a_h[A_RUNS];
#pragma unroll
    for (int v = 0; v < A_RUNS; ++v) {
        const int c = tid + v * THREADS;  // run c: row c / 2, k half c % 2
        a_row[v] = c >> 1;
        a_h[v] = c & 1;
        a_src[v] = g.A + (int64_t)min(m0 + a_row[v], M - 1) * g.lda + 8 * a_h[v];
    }
    const float *b_src[B_RUNS];
    int b_col[B_RUNS], b_h[B_RUNS];
#pragma unroll
    for (int v = 0; v < B_RUNS; ++v) {
        const int c = tid + v * THREADS;  // run c: column c % BN, k half c / BN
        b_col[v] = c % BN;
        b_h[v] = c / BN;
        b_src[v] = g.B + (int64_t)(8 * b_h[v]) * g.ldb + min(n0 + b_col[v], N - 1);
    }

    // Two register slots of fetched windows.
    f32x8 ra[2][A_RUNS], rb[2][B_RUNS];

    // Window w (k = 16w .. 16w+15) into slot s.  FULL: every k < K.
    auto fetch = [&](auto full_tag, int s, int w) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int64_t k0 = (int64_t)w * BK;
#pragma unroll
        for (int v = 0; v < A_RUNS; ++v) {
            const float *p = a_src[v] + k0;
            if constexpr (FULL) {
                const f32x4 lo = load16(p), hi = load16(p + 4);
                ra[s][v] = f32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            } else {
                const int64_t kk = k0 + 8 * a_h[v];
#pragma unroll
                for (int e = 0; e < 8; ++e) ra[s][v][e] = kk + e < K ? p[e] : 0.0f;
            }
        }
#pragma unroll
        for (int v = 0; v < B_RUNS; ++v) {
            const float *p = b_src[v] + k0 * g.ldb;
            const int64_t kk = k0 + 8 * b_h[v];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (FULL) {
                    rb[s][v][e] = p[(int64_t)e * g.ldb];
                } else {
                    rb[s][v][e] = kk + e < K ? p[(int64_t)e * g.ldb] : 0.0f;
                }
            }
        }
    };
    // Split slot s into parts and store them in LDS stage `stage`.
    auto stash = [&](int s, int stage) {
        __bf16 *base = lds + stage * STAGE;
#pragma unroll
        for (int v = 0; v < A_RUNS; ++v) {
            bf16x8 p[3];
            split3(ra[s][v], p[0], p[1], p[2]);
#pragma unroll
            for (int q = 0; q < PARTS; ++q)
                *(bf16x8 *)(base + q * A_PART + slot(a_row[v], a_h[v])) = p[q];
        }
#pragma unroll
        for (int v = 0; v < B_RUNS; ++v) {
            bf16x8 p[3];
            split3(rb[s][v], p[0], p[1], p[2]);
#pragma unroll
            for (int q = 0; q < PARTS; ++q)
                *(bf16x8 *)(base + PARTS * A_PART + q * B_PART + slot(b_col[v], b_h[v])) = p[q];
        }
    };

    struct Frag {
        bf16x8 a[PARTS][TM];
        bf16x8 b[PARTS][TN];
    };
    auto read_frag = [&](Frag &f, int stage) {
        const __bf16 *base = lds + stage * STAGE;
#pragma unroll
        for (int q = 0; q < PARTS; ++q) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                f.a[q][i] = *(const bf16x8 *)(base + q * A_PART + slot(wm * WM + 32 * i + lr, lh));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                f.b[q][j] = *(const bf16x8 *)(base + PARTS * A_PART + q * B_PART +
                                              slot(wn * WN + 32 * j + lr, lh));
        }
    };
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
    auto multiply = [&](const Frag &f) {
#pragma unroll
        for (int t = 0; t < 6; ++t)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        f.a[PP[t][0]][i], f.b[PP[t][1]][j], acc[i][j], 0, 0, 0);
    };

    const int nw = (K + BK - 1) / BK;   // windows
    const int nfull = K / BK;           // windows with every k < K
    auto fetch_any = [&](int s, int w) {
        if (w < nfull) {
            fetch(std::true_type{}, s, w);
        } else if (w < nw) {
            fetch(std::false_type{}, s, w);
        }
    };

    // Prologue: windows 0 and 1 to LDS, windows 2 and 3 to the register slots.
    fetch_any(0, 0);
    stash(0, 0);
    if (1 < nw) {
        fetch_any(1, 1);
        stash(1, 1);
    }
    fetch_any(0, 2);
    fetch_any(1, 3);
    __syncthreads();
    Frag frag[2];
    read_frag(frag[0], 0);

    // Window w: its fragments are in frag[w & 1]; LDS holds w and w + 1; the
    // register slots hold w + 2 (slot w & 1) and w + 3.
    auto body = [&](auto steady_tag, auto slot_tag, int w) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        constexpr int S = decltype(slot_tag)::value;
        const int cur = w % STAGES;
        const int next = cur + 1 == STAGES ? 0 : cur + 1;
        const int fill = cur == 0 ? STAGES - 1 : cur - 1;
        read_frag(frag[S ^ 1], next);  // unused after the last window; keeps waits exact
        if (STEADY || w + 2 < nw) stash(S, fill);
        if constexpr (STEADY) {
            fetch(std::true_type{}, S, w + 4);
        } else {
            fetch_any(S, w + 4);
        }
        multiply(frag[S]);
        if constexpr (STEADY) {
            // MFMAs spread between the memory operations (see interleave()).
            interleave<6 * TM * TN, PARTS * (TM + TN), PARTS * (A_RUNS + B_RUNS),
                       2 * A_RUNS + 8 * B_RUNS>();
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };

    int w = 0;
    // Steady state: windows up to w + 5 all full, two at a time (the register slot
    // of a window is static in the unrolled body).
    for (; w + 5 < nfull; w += 2) {
        body(std::true_type{}, std::integral_constant<int, 0>{}, w);
        body(std::true_type{}, std::integral_constant<int, 1>{}, w + 1);
    }
    for (; w < nw; w += 2) {
        body(std::false_type{}, std::integral_constant<int, 0>{}, w);
        if (w + 1 < nw) body(std::false_type{}, std::integral_constant<int, 1>{}, w + 1);
    }

    // Epilogue (same accumulator layout as the fp32 rung).
    const float alpha = g.alpha, beta = g.beta;
    const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WM + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (!full && row >= M) continue;
            float *dst = g.C + (int64_t)row * g.ldc;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n0 + wn * WN + 32 * j + lr;
                if (full || col < N) dst[col] = epilogue(acc[i][j][r], alpha, beta, dst + col);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace split

hipError_t launch_split(const Problem &p, hipStream_t s) {
    if (p.ta || p.tb) return hipErrorInvalidValue;
    const int64_t tiles_m = (p.M + split::BM - 1) / split::BM;
    const int64_t tiles_n = (p.N + split::BN - 1) / split::BN;
    if (tiles_m * tiles_n > INT32_MAX) return hipErrorInvalidValue;
    const split::Args g{p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.alpha, p.beta};
    return launch(split::split_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(split::THREADS), 0,
                  s, g, (int)tiles_m, (int)tiles_n);
}

}  // namespace sgemm
