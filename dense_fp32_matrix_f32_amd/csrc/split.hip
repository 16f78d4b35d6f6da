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
// Layout of the work follows the fp32 rung (mfma_kernel.h): a block of C per
// work-group (256 x 256 or 256 x 128), eight waves (two per SIMD, so that one
// wave's part splitting and LDS waits overlap the other's MFMAs), k windows of
// 16 in a three-stage LDS ring with one barrier per window.  Global loads run
// ahead into registers; the split into parts happens when a window goes from
// registers to LDS, so each value is split once per work-group.  Both operands are kept in
// LDS with k contiguous (B is gathered column by column from global memory), as
// rows of 16 bf16 per part whose two 16-byte halves swap places on every other
// group of 8 rows, which keeps the fragment reads free of bank conflicts.
// v_mfma_f32_32x32x16_bf16: lane l supplies row (column) l % 32 and eight
// consecutive k starting at 8*(l / 32), the same k for A and B.
#include <cmath>

#include "mfma_kernel.h"

namespace sgemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

namespace split {

constexpr int BK = 16;
constexpr int PARTS = 3;

// BM x BN block of C per work-group, WM x WN per wave, STAGES LDS buffers, OCC
// work-groups per CU that the register allocation must allow.
// FRAGS: 2 reads the next window's fragments during the current one's MFMAs
// (one wave per SIMD); 1 reads each window's fragments at its start and leaves
// the wait to be covered by the other waves of the SIMD (fewer registers); 0
// does the same for A and reads the parts of B one at a time between the MFMAs
// that use them (fewer registers still).
// SLOTS: windows held in registers between their global loads and their LDS
// stores (the loads run 2 + SLOTS windows ahead of the MFMAs).
// RUN: consecutive k (4 or 8) of one row of A or column of B that a work-item
// loads, splits and stores as one piece.
template <int BM_, int BN_, int WM_, int WN_, int STAGES_ = 3, int OCC_ = 1, int GROUP_M_ = 8,
          int FRAGS_ = 2, int SLOTS_ = 2, int RUN_ = 8>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
    static constexpr int OCC = OCC_, GROUP_M = GROUP_M_, FRAGS = FRAGS_, SLOTS = SLOTS_;
    static constexpr int RUN = RUN_;
    static_assert(FRAGS >= 0 && FRAGS <= 2, "fragment buffers");
    static_assert(SLOTS == 1 || SLOTS == 2, "register slots");
    static_assert(RUN == 4 || RUN == 8, "runs of 4 or 8 k");
    static constexpr int TM = WM / 32, TN = WN / 32;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int THREADS = (BM / WM) * WAVES_N * 64;
    // bf16 elements of one part of one operand window, and of one LDS stage
    static constexpr int A_PART = BM * BK, B_PART = BN * BK;
    static constexpr int STAGE = PARTS * (A_PART + B_PART);
    // global -> register work per thread and window: A as runs of RUN k of one
    // row, B as runs of RUN k of one column
    static constexpr int A_RUNS = BM * BK / RUN / THREADS;
    static constexpr int B_RUNS = BN * BK / RUN / THREADS;
    static constexpr int RPR = BK / RUN;  // runs per row (column)
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "wave tiling");
    static_assert(A_RUNS >= 1 && B_RUNS >= 1 && A_RUNS * THREADS * RUN == BM * BK &&
                      B_RUNS * THREADS * RUN == BN * BK,
                  "whole runs");
    static_assert(STAGES == 3, "three-stage ring");
    static_assert(STAGES * STAGE * 2 <= 160 * 1024, "LDS budget");
};

// Element offset (bf16 units) of element k of row `row` in a part: the two
// 8-wide halves of a row swap places on every other group of 8 rows.
__device__ __forceinline__ int slot(int row, int k) {
    return row * BK + 8 * ((k >> 3) ^ ((row >> 3) & 1)) + (k & 7);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// bf16 pair (round to nearest even, v_cvt_pk_bf16_f32) as one 32-bit word.
__device__ __forceinline__ unsigned to_bf16x2(float x, float y) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x, y}, bf16x2));
}

// The three bf16 parts of eight floats (see the file comment), two at a time:
// the value of a part is read back from its bits, so each pair needs one
// conversion per part.  An infinite input leaves NaN residuals.
template <int R> struct Run;
template <> struct Run<8> {
    typedef f32x8 f;
    typedef bf16x8 b;
    typedef u32x4 u;
};
template <> struct Run<4> {
    typedef f32x4 f;
    typedef __bf16 b __attribute__((ext_vector_type(4)));
    typedef unsigned u __attribute__((ext_vector_type(2)));
};

template <int R>
__device__ __forceinline__ void split3(const typename Run<R>::f &x, typename Run<R>::b &p0,
                                       typename Run<R>::b &p1, typename Run<R>::b &p2) {
    typename Run<R>::u w0, w1, w2;
#pragma unroll
    for (int e = 0; e < R / 2; ++e) {
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
    p0 = __builtin_bit_cast(typename Run<R>::b, w0);
    p1 = __builtin_bit_cast(typename Run<R>::b, w1);
    p2 = __builtin_bit_cast(typename Run<R>::b, w2);
}

// Scheduling hint for the steady-state body: each of its MF MFMAs is followed by
// at most one memory instruction (the DSR LDS reads, then the DSW LDS writes,
// then the VMR global loads) and up to VPS vector-ALU instructions (the splits),
// so the matrix cores keep running while the parts are computed.  Bodies with
// fewer MFMAs than memory instructions are left to the default scheduler.
template <int MF, int DSR, int DSW, int VMR, int VPS>
__device__ __forceinline__ void interleave_split() {
    if constexpr (MF >= DSR + DSW + VMR) {
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i < DSR) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        } else if (i < DSR + DSW) {
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
        } else if (i < DSR + DSW + VMR) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        }
        __builtin_amdgcn_sched_group_barrier(0x002, VPS, 0);    // vector ALU
    }
    }
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

// Loads through a buffer resource whose base is the uniform address `base`, at
// byte offset voff + soff (voff per lane, soff uniform); no range limit, the
// caller keeps every access inside its matrix.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const char *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, -1, 0x00020000);
}

// NARROW: every per-lane byte offset from the block's first row of A or first
// column of B stays below 2^31 (checked on the host), so full windows are read
// with buffer loads: uniform bases advanced once per window, fixed lane offsets,
// and for B the k rows of a run as uniform offsets, with no vector address
// arithmetic.  Otherwise every lane keeps 64-bit pointers.
template <class T, bool NARROW>
__global__ __launch_bounds__(T::THREADS, T::OCC) void split_kernel(Args g, int tiles_m,
                                                                  int tiles_n) {
    constexpr int BM = T::BM, BN = T::BN, WM = T::WM, WN = T::WN, TM = T::TM, TN = T::TN;
    constexpr int THREADS = T::THREADS, WAVES_N = T::WAVES_N, STAGES = T::STAGES;
    constexpr int A_PART = T::A_PART, B_PART = T::B_PART, STAGE = T::STAGE;
    constexpr int A_RUNS = T::A_RUNS, B_RUNS = T::B_RUNS;
    __shared__ __attribute__((aligned(16))) __bf16 lds[STAGES * STAGE];
    const int M = g.M, N = g.N, K = g.K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    tile_order(blockIdx.x, tiles_m, tiles_n, T::GROUP_M, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- global -> register assignment ----
    constexpr int RUN = T::RUN, RPR = T::RPR;
    typedef typename Run<RUN>::f fR;
    typedef typename Run<RUN>::b bR;
    const float *a_src[A_RUNS];
    uint32_t a_off[A_RUNS];  // byte offset of a_src[v] from a_org
    int a_row[A_RUNS], a_k[A_RUNS];
    const char *a_org = (const char *)(g.A + (int64_t)m0 * g.lda);
#pragma unroll
    for (int v = 0; v < A_RUNS; ++v) {
        const int c = tid + v * THREADS;  // run c: row c / RPR, k RUN * (c % RPR)
        a_row[v] = c / RPR;
        a_k[v] = RUN * (c % RPR);
        const int64_t e = (int64_t)(min(m0 + a_row[v], M - 1) - m0) * g.lda + a_k[v];
        a_src[v] = g.A + (int64_t)m0 * g.lda + e;
        a_off[v] = (uint32_t)(e * 4);
    }
    const float *b_src[B_RUNS];
    uint32_t b_off[B_RUNS];  // byte offset of b_src[v] from b_org
    int b_col[B_RUNS], b_k[B_RUNS];
    const char *b_org = (const char *)(g.B + n0);
#pragma unroll
    for (int v = 0; v < B_RUNS; ++v) {
        const int c = tid + v * THREADS;  // run c: column c % BN, k RUN * (c / BN)
        b_col[v] = c % BN;
        b_k[v] = RUN * (c / BN);
        const int64_t e = (int64_t)b_k[v] * g.ldb + (min(n0 + b_col[v], N - 1) - n0);
        b_src[v] = g.B + n0 + e;
        b_off[v] = (uint32_t)(e * 4);
    }

    // Register slots of fetched windows.
    fR ra[T::SLOTS][A_RUNS], rb[T::SLOTS][B_RUNS];

    // Window w (k = 16w .. 16w+15) into slot s.  FULL: every k < K.
    auto fetch = [&](auto full_tag, int s, int w) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int64_t k0 = (int64_t)w * BK;
        if constexpr (FULL && NARROW) {
            const __amdgpu_buffer_rsrc_t ra_ = rsrc_at(a_org + k0 * 4);
            const __amdgpu_buffer_rsrc_t rb_ = rsrc_at(b_org + k0 * g.ldb * 4);
#pragma unroll
            for (int v = 0; v < A_RUNS; ++v)
#pragma unroll
                for (int e4 = 0; e4 < RUN / 4; ++e4) {
                    const f32x4 q = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra_, a_off[v] + 16 * e4, 0, 0));
                    ra[s][v][4 * e4 + 0] = q.x;
                    ra[s][v][4 * e4 + 1] = q.y;
                    ra[s][v][4 * e4 + 2] = q.z;
                    ra[s][v][4 * e4 + 3] = q.w;
                }
#pragma unroll
            for (int v = 0; v < B_RUNS; ++v)
#pragma unroll
                for (int e = 0; e < RUN; ++e)
                    rb[s][v][e] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(rb_, b_off[v],
                                                                    (int)(e * g.ldb * 4), 0));
            return;
        }
#pragma unroll
        for (int v = 0; v < A_RUNS; ++v) {
            const float *p =
                (NARROW ? (const float *)(a_org + a_off[v]) : a_src[v]) + k0;
            if constexpr (FULL) {
#pragma unroll
                for (int e4 = 0; e4 < RUN / 4; ++e4) {
                    const f32x4 q = load16(p + 4 * e4);
                    ra[s][v][4 * e4 + 0] = q.x;
                    ra[s][v][4 * e4 + 1] = q.y;
                    ra[s][v][4 * e4 + 2] = q.z;
                    ra[s][v][4 * e4 + 3] = q.w;
                }
            } else {
                const int64_t kk = k0 + a_k[v];
#pragma unroll
                for (int e = 0; e < RUN; ++e) ra[s][v][e] = kk + e < K ? p[e] : 0.0f;
            }
        }
#pragma unroll
        for (int v = 0; v < B_RUNS; ++v) {
            const float *p =
                (NARROW ? (const float *)(b_org + b_off[v]) : b_src[v]) + k0 * g.ldb;
            const int64_t kk = k0 + b_k[v];
#pragma unroll
            for (int e = 0; e < RUN; ++e) {
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
            bR p[3];
            split3<RUN>(ra[s][v], p[0], p[1], p[2]);
#pragma unroll
            for (int q = 0; q < PARTS; ++q)
                *(bR *)(base + q * A_PART + slot(a_row[v], a_k[v])) = p[q];
        }
#pragma unroll
        for (int v = 0; v < B_RUNS; ++v) {
            bR p[3];
            split3<RUN>(rb[s][v], p[0], p[1], p[2]);
#pragma unroll
            for (int q = 0; q < PARTS; ++q)
                *(bR *)(base + PARTS * A_PART + q * B_PART + slot(b_col[v], b_k[v])) = p[q];
        }
    };

    struct Frag {
        bf16x8 a[PARTS][TM];
        bf16x8 b[PARTS][TN];
    };
    auto read_b = [&](bf16x8 *b, const __bf16 *base, int q) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
            b[j] = *(const bf16x8 *)(base + PARTS * A_PART + q * B_PART +
                                     slot(wn * WN + 32 * j + lr, 8 * lh));
    };
    auto read_frag = [&](Frag &f, int stage) {
        const __bf16 *base = lds + stage * STAGE;
#pragma unroll
        for (int q = 0; q < PARTS; ++q) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                f.a[q][i] = *(const bf16x8 *)(base + q * A_PART + slot(wm * WM + 32 * i + lr, 8 * lh));
            if constexpr (T::FRAGS > 0) read_b(f.b[q], base, q);
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

    // FRAGS == 0: the parts of B in turn, each followed by its products,
    // (0,2), (1,1), (0,1), (2,0), (1,0), (0,0).
    auto multiply_stream = [&](const Frag &f, int stage) {
        const __bf16 *base = lds + stage * STAGE;
#pragma unroll
        for (int q = PARTS - 1; q >= 0; --q) {
            bf16x8 b[TN];
            read_b(b, base, q);
#pragma unroll
            for (int p = 0; p + q < PARTS; ++p) {
                const int pa = q == 0 ? PARTS - 1 - p : p;  // with B part 0, A parts 2, 1, 0
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[pa][i], b[j],
                                                                            acc[i][j], 0, 0, 0);
            }
        }
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

    // Prologue: windows 0 and 1 to LDS, windows 2 .. 1 + SLOTS to the register slots.
    constexpr int AHEAD = 2 + T::SLOTS;  // distance from the computed to the fetched window
    fetch_any(0, 0);
    stash(0, 0);
    if (1 < nw) {
        fetch_any(0, 1);
        stash(0, 1);
    }
#pragma unroll
    for (int s2 = 0; s2 < T::SLOTS; ++s2) fetch_any(s2, 2 + s2);
    __syncthreads();
    Frag frag[T::FRAGS == 2 ? 2 : 1];
    if constexpr (T::FRAGS == 2) read_frag(frag[0], 0);

    // Window w (parity P = w & 1): LDS holds w and w + 1; register slot
    // (w + 2) % SLOTS holds w + 2; with two fragment buffers, frag[P] holds w's.
    auto body = [&](auto steady_tag, auto parity_tag, int w) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        constexpr int P = decltype(parity_tag)::value;
        constexpr int S = P % T::SLOTS;
        const int cur = w % STAGES;
        const int next = cur + 1 == STAGES ? 0 : cur + 1;
        const int fill = cur == 0 ? STAGES - 1 : cur - 1;
        if constexpr (T::FRAGS == 2) {
            read_frag(frag[P ^ 1], next);  // unused after the last window; keeps waits exact
        } else {
            read_frag(frag[0], cur);
        }
        if (STEADY || w + 2 < nw) stash(S, fill);
        if constexpr (STEADY) {
            fetch(std::true_type{}, S, w + AHEAD);
        } else {
            fetch_any(S, w + AHEAD);
        }
        if constexpr (T::FRAGS == 0) {
            multiply_stream(frag[0], cur);
        } else {
            multiply(frag[T::FRAGS == 2 ? P : 0]);
        }
        if constexpr (STEADY && T::FRAGS > 0) {
            interleave_split<6 * TM * TN, PARTS * (TM + TN), PARTS * (A_RUNS + B_RUNS),
                             RUN / 4 * A_RUNS + RUN * B_RUNS, 4>();
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };

    int w = 0;
    // Steady state: every window fetched in the pair is full; two windows at a
    // time, so that slots and fragment buffers are static in the unrolled body.
    for (; w + 1 + AHEAD < nfull; w += 2) {
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

template <class T>
hipError_t launch_split_tile(const Problem &p, hipStream_t s) {
    if (p.ta || p.tb) return hipErrorInvalidValue;
    const int64_t tiles_m = (p.M + T::BM - 1) / T::BM;
    const int64_t tiles_n = (p.N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > INT32_MAX) return hipErrorInvalidValue;
    const Args g{p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.alpha, p.beta};
    // largest lane offsets: the last row of A's block plus a window, the last k
    // row of B's window plus a row of the block
    const bool narrow = (((int64_t)(T::BM - 1) * p.lda + BK) * 4 < ((int64_t)1 << 31)) &&
                        (((int64_t)(BK - 1) * p.ldb + T::BN) * 4 < ((int64_t)1 << 31));
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(T::THREADS);
    if (narrow)
        return launch(split_kernel<T, true>, grid, block, 0, s, g, (int)tiles_m, (int)tiles_n);
    return launch(split_kernel<T, false>, grid, block, 0, s, g, (int)tiles_m, (int)tiles_n);
}

// 256 x 256 blocks of eight waves (two per SIMD) with 128 x 64 of C each; B
// parts read one at a time: large products.
using SplitHuge = Tile<256, 256, 128, 64, 3, 1, 8, 0, 1, 8>;
// 256 x 128 blocks of eight waves with 64 x 64 each, runs of 4 k: grids of about
// one block per CU, such as 2048 x 3072.
using SplitMid = Tile<256, 128, 64, 64, 3, 1, 8, 1, 1, 4>;

}  // namespace split

// The busiest CU works through ceil(blocks / CUs) blocks; each costs BM*BN / e
// with e the configuration's measured throughput at 8192^3 (233 and 208
// TFLOP/s).  The cheaper estimate wins.
hipError_t launch_split(const Problem &p, hipStream_t s) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    auto cost = [&](int bm, int bn, double e) {
        const double blocks = (double)((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
        return std::ceil(blocks / cus) * bm * bn / e;
    };
    if (cost(split::SplitHuge::BM, split::SplitHuge::BN, 233.0) <=
        cost(split::SplitMid::BM, split::SplitMid::BN, 208.0))
        return split::launch_split_tile<split::SplitHuge>(p, s);
    return split::launch_split_tile<split::SplitMid>(p, s);
}

}  // namespace sgemm
