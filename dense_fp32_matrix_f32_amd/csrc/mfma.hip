// mfma.hip -- register-blocked fp32 matrix-core rung of the ladder.
//
// Same decomposition as the pages' tiled kernel (page "CUDA算子优化(4)：矩阵乘法",
// section "版本V1共享内存分块": each work-group owns a TILE_M x TILE_N block of C and
// slides a TILE_K window along k, staging the A and B windows in on-chip memory),
// re-sized for gfx950:
//   * a BM x BN block of C per work-group, BK-wide k windows in a ring of two or
//     three LDS stages (later windows are written while the current one is read,
//     so one barrier per window replaces the pages' two);
//   * global -> LDS copies as 16-byte loads, issued a window ahead into
//     registers so that their latency overlaps a whole window of math;
//   * the operand fragments of the next 8-wide k step are read from LDS while
//     the MFMAs of the current step run; with three stages this reaches across
//     the window boundary, so the barrier does not leave the matrix cores idle;
//   * each wave owns a WM x WN sub-block held as (WM/32) x (WN/32) accumulators
//     of v_mfma_f32_32x32x2f32 (full fp32 inputs, fp32 accumulation, 4096 flops
//     per instruction), which is where the per-element fused multiply-adds of
//     the pages' kernels go;
//   * optionally KW groups of waves split each window's k range between them
//     and add their partial blocks through LDS at the end, in a fixed order, so
//     a small block of C still keeps all four SIMDs of a CU busy;
//   * work-group ids are re-ordered so that each XCD works on one compact region
//     of C (see tile_order.h).
//
// Operand placement.  The k order inside one MFMA is fixed by the hardware.
// Across the four MFMAs of an 8-wide k step, lane half h supplies
// k = k8 + 4h + q to the q-th instruction, so each lane fetches four
// consecutive k of A with one 16-byte LDS read.  In the n direction lane c of
// accumulator block j stands for column TN*c + j of the wave's strip, so a lane
// fetches its TN columns of B for one k with one LDS read, and later stores TN
// adjacent results of C.  A and B use the same k assignment, so every product
// A[i][k]*B[k][j] is formed exactly once.
//
// Edges: rows of A beyond M and columns of B beyond N are read from the last
// valid row/column (they only feed outputs that are not stored); the last,
// partial k window is zero-filled on both operands (the pages' zero-fill of
// partial tiles), so no value outside the logical matrices enters a stored
// result and no load leaves the matrices' extents.
#include <cmath>
#include <type_traits>

#include "internal.h"

namespace sgemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int N> struct VecOf;
template <> struct VecOf<1> { typedef float type; };
template <> struct VecOf<2> { typedef f32x2 type; };
template <> struct VecOf<4> { typedef f32x4 type; };
// Three adjacent floats, 4-byte aligned: read from LDS as a two-dword and a
// one-dword access.
struct F3 {
    float e[3];
};
template <> struct VecOf<3> { typedef F3 type; };

template <int N>
__device__ __forceinline__ float lane_of(const typename VecOf<N>::type &v, int j) {
    if constexpr (N == 1) {
        return v;
    } else if constexpr (N == 3) {
        return v.e[j];
    } else {
        return v[j];
    }
}

// 16-byte load from a 4-byte aligned address (gfx950 global memory instructions
// accept dword-aligned multi-dword accesses).
__device__ __forceinline__ f32x4 load16(const float *p) {
    f32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// BM x BN block of C per work-group, BK-wide k windows, WM x WN block per wave,
// KW wave groups splitting k, GROUP_M tile-rows per ordering group, STAGES LDS
// buffers (2 or 3), and OCC the number of waves per SIMD that the register
// allocation must allow.
// Scheduling hint for one basic block holding MF MFMAs, DSR LDS reads, DSW LDS
// writes and VMR global loads: each memory instruction is placed right after an
// MFMA, so a single wave keeps its matrix core fed while it issues them.  When
// there are fewer MFMAs than memory instructions the block is left to the
// default scheduler.
template <int MF, int DSR, int DSW, int VMR>
__device__ __forceinline__ void interleave() {
    if constexpr (MF >= DSR + DSW + VMR) {
#pragma unroll
        for (int i = 0; i < DSR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
#pragma unroll
        for (int i = 0; i < DSW; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
        }
#pragma unroll
        for (int i = 0; i < VMR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        }
        if constexpr (MF > DSR + DSW + VMR)
            __builtin_amdgcn_sched_group_barrier(0x008, MF - DSR - DSW - VMR, 0);
    }
}

template <int BM_, int BN_, int BK_, int WM_, int WN_, int KW_, int GROUP_M_, int STAGES_ = 2,
          int OCC_ = 1, int PAD_A_ = 4, int PAD_B_ = 8>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, KW = KW_;
    static constexpr int GROUP_M = GROUP_M_, STAGES = STAGES_, OCC = OCC_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int SPATIAL = WAVES_M * WAVES_N;    // waves per k group
    static constexpr int THREADS = SPATIAL * KW * 64;
    static constexpr int TM = WM / 32, TN = WN / 32;     // 32x32 accumulators per wave
    static constexpr int ACC = TM * TN * 16;             // accumulator floats per lane
    static constexpr int PA = BK + PAD_A_;               // A row pitch in LDS (floats)
    static constexpr int PB = BN + PAD_B_;               // B row pitch in LDS (floats)
    static constexpr int A_STAGE = BM * PA, B_STAGE = BK * PB;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int RED = (KW - 1) * SPATIAL * 64 * ACC;  // split-k partials
    static constexpr int LDS_FLOATS = STAGES * STAGE > RED ? STAGES * STAGE : RED;
    static constexpr int A_TOTAL = BM * BK / 4, B_TOTAL = BK * BN / 4;  // 16-byte vectors
    static constexpr int A_VECS = (A_TOTAL + THREADS - 1) / THREADS;     // per thread
    static constexpr int B_VECS = (B_TOTAL + THREADS - 1) / THREADS;
    static constexpr int STEPS = BK / (8 * KW);          // 8-wide k steps per group per window
    static constexpr int MF = 4 * TM * TN;               // MFMAs per step
    static constexpr int DSR = TM + 4 * (TN == 3 ? 2 : 1);  // LDS reads per step
    static constexpr int DSW = A_VECS + B_VECS;          // LDS writes per window
    static constexpr int VMR = A_VECS + B_VECS;          // global loads per window
    // The steady-state loop writes LDS in the first step of a window and issues
    // the `vmr` global loads of a later window in the same step, or in the second
    // step when one step has too few MFMAs to cover all of those memory
    // instructions.
    static constexpr int load_step(int vmr) {
        return (STEPS > 1 && MF < DSR + DSW + vmr) ? 1 : 0;
    }
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0, "wave tiling");
    static_assert(TN >= 1 && TN <= 4, "a lane holds 1 to 4 adjacent columns");
    static_assert(BK % (8 * KW) == 0 && BK % 4 == 0, "k window splits into 8-wide steps");
    static_assert(THREADS <= 1024, "work-group size");
    static_assert(PAD_A_ % 4 == 0 && PAD_B_ % 4 == 0, "16-byte aligned LDS rows");
    static_assert(STAGES == 2 || (STAGES == 3 && STEPS % 2 == 0),
                  "a three-stage ring carries fragments across windows in an even step count");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");
};

// The operands of one product.
struct GemmArgs {
    int M, N, K;
    const float *__restrict__ A;
    int64_t lda;
    const float *__restrict__ B;
    int64_t ldb;
    float *__restrict__ C;
    int64_t ldc;
};

template <class T>
using Acc = f32x16[T::TM][T::TN];

// acc += the product of A rows m0..m0+BM-1 and B columns n0..n0+BN-1 over the
// k windows [w_begin, w_end) (window w covers k = w*BK .. w*BK+BK-1).  Called by
// every work-item of the group; uses all of `lds` and ends on a barrier, so LDS
// is free again when it returns.
template <class T>
__device__ __forceinline__ void mma_tile(const GemmArgs &g, float *lds, int m0, int n0,
                                         int w_begin, int w_end, Acc<T> &acc) {
    typedef typename VecOf<T::TN>::type BVec;
    const int M = g.M, N = g.N, K = g.K;
    const int64_t lda = g.lda, ldb = g.ldb;
    const float *__restrict__ A = g.A;
    const float *__restrict__ B = g.B;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int kg = wave / T::SPATIAL, sw = wave % T::SPATIAL;
    const int wm = sw / T::WAVES_N, wn = sw % T::WAVES_N;

    // ---- global-load assignment (fixed for the whole k loop) ----
    constexpr int AQ = T::BK / 4;  // 16-byte vectors per A row of the window
    constexpr int BQ = T::BN / 4;  // 16-byte vectors per B row of the window
    // Vector v of this work-item exists iff tid + v*THREADS < TOTAL; only the last
    // one can be missing, and only when TOTAL is not a multiple of THREADS.  A
    // missing vector re-reads the last one (in bounds) and is not stored.
    auto has_a = [&](int v) {
        return (T::A_TOTAL % T::THREADS == 0) || tid + v * T::THREADS < T::A_TOTAL;
    };
    auto has_b = [&](int v) {
        return (T::B_TOTAL % T::THREADS == 0) || tid + v * T::THREADS < T::B_TOTAL;
    };
    const float *a_src[T::A_VECS];
    int a_lds[T::A_VECS], a_k[T::A_VECS];
#pragma unroll
    for (int v = 0; v < T::A_VECS; ++v) {
        const int c = min(tid + v * T::THREADS, T::A_TOTAL - 1);
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
        const int c = min(tid + v * T::THREADS, T::B_TOTAL - 1);
        const int r = c / BQ, q = c % BQ;
        b_k[v] = r;
        b_n[v] = n0 + q * 4;
        b_src[v] = B + (int64_t)r * ldb + n0 + q * 4;
        b_lds[v] = T::A_STAGE + r * T::PB + q * 4;
    }

    f32x4 ra[T::A_VECS], rb[T::B_VECS];

    // Loads of the k window starting at k0 into registers.  Work-groups whose
    // columns all lie inside B (every one but the last column of tiles) take the
    // plain 16-byte path for every vector; the test is uniform across the group.
    const bool cols_inside = n0 + T::BN <= N;
    auto fetch = [&](int k0) {
        if (k0 + T::BK <= K) {
#pragma unroll
            for (int v = 0; v < T::A_VECS; ++v) ra[v] = load16(a_src[v] + k0);
            if (cols_inside) {
#pragma unroll
                for (int v = 0; v < T::B_VECS; ++v) rb[v] = load16(b_src[v] + (int64_t)k0 * ldb);
            } else {
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
        for (int v = 0; v < T::A_VECS; ++v)
            if (has_a(v)) *(f32x4 *)(s + a_lds[v]) = ra[v];
#pragma unroll
        for (int v = 0; v < T::B_VECS; ++v)
            if (has_b(v)) *(f32x4 *)(s + b_lds[v]) = rb[v];
    };

    const int a_frag = (wm * T::WM + lr) * T::PA + 4 * lh;
    const int b_frag = T::A_STAGE + (4 * lh) * T::PB + wn * T::WN + T::TN * lr;

    // Fragments of one 8-wide k step: four consecutive k of TM row blocks of A and,
    // for each of those k, TN adjacent columns of B.
    struct Frag {
        f32x4 a[T::TM];
        BVec b[4];
    };
    auto read_frag = [&](Frag &f, const float *s, int t) {
        const int k8 = (t * T::KW + kg) * 8;
#pragma unroll
        for (int i = 0; i < T::TM; ++i) f.a[i] = *(const f32x4 *)(s + a_frag + i * 32 * T::PA + k8);
#pragma unroll
        for (int q = 0; q < 4; ++q) f.b[q] = *(const BVec *)(s + b_frag + (k8 + q) * T::PB);
    };
    auto multiply = [&](const Frag &f) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        f.a[i][q], lane_of<T::TN>(f.b[q], j), acc[i][j], 0, 0, 0);
    };

    // Prologue: the first STAGES-1 windows go to LDS, the next one to registers.
    fetch(w_begin * T::BK);
    stash(0);
    if constexpr (T::STAGES == 3) {
        if (w_begin + 1 < w_end) {
            fetch((w_begin + 1) * T::BK);
            stash(1);
        }
    }
    __syncthreads();
    if (w_begin + T::STAGES - 1 < w_end) fetch((w_begin + T::STAGES - 1) * T::BK);

    Frag frag[2];
    int cur = 0;  // LDS stage of window w
    int w = w_begin;
    if constexpr (T::STAGES == 3) read_frag(frag[0], lds, 0);

    // Steady state: a window whose successors up to w + STAGES are all full.
    // The body has no branches, so the copies of later windows (LDS stores of
    // window w + STAGES - 1, global loads of window w + STAGES) and the fragment
    // reads of the next step are spread one by one between the MFMAs instead of
    // stalling the matrix cores in a block of their own.  Work-groups on the
    // right edge of C (EDGE) load B one element at a time with the column index
    // clamped to N - 1, which keeps the body free of branches there too.
    auto steady = [&](auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        constexpr int VMR = EDGE ? T::A_VECS + 4 * T::B_VECS : T::VMR;
        constexpr int LOAD_STEP = T::load_step(VMR);
        int b_off[T::B_VECS][4];
        if constexpr (EDGE) {
#pragma unroll
            for (int v = 0; v < T::B_VECS; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) b_off[v][e] = min(b_n[v] + e, N - 1) - b_n[v];
        }
        const int steady_end = min(w_end, K / T::BK) - T::STAGES;
        for (; w < steady_end; ++w) {
            const float *s = lds + cur * T::STAGE;
            const int next = cur + 1 == T::STAGES ? 0 : cur + 1;
            const int fill = cur == 0 ? T::STAGES - 1 : cur - 1;
            if constexpr (T::STAGES == 2) read_frag(frag[0], s, 0);
#pragma unroll
            for (int t = 0; t < T::STEPS; ++t) {
                if (t + 1 < T::STEPS) {
                    read_frag(frag[(t + 1) & 1], s, t + 1);
                } else if constexpr (T::STAGES == 3) {
                    read_frag(frag[(t + 1) & 1], lds + next * T::STAGE, 0);
                }
                if (t == 0) stash(fill);
                if (t == LOAD_STEP) {
                    const int64_t k0 = (int64_t)(w + T::STAGES) * T::BK;
#pragma unroll
                    for (int v = 0; v < T::A_VECS; ++v) ra[v] = load16(a_src[v] + k0);
#pragma unroll
                    for (int v = 0; v < T::B_VECS; ++v) {
                        const float *p = b_src[v] + k0 * ldb;
                        if constexpr (EDGE) {
                            rb[v].x = p[b_off[v][0]];
                            rb[v].y = p[b_off[v][1]];
                            rb[v].z = p[b_off[v][2]];
                            rb[v].w = p[b_off[v][3]];
                        } else {
                            rb[v] = load16(p);
                        }
                    }
                }
                multiply(frag[t & 1]);
                // LDS reads issued in step 0, in a middle step and in the last step.
                constexpr int R0 = (1 < T::STEPS || T::STAGES == 3) ? T::DSR : 0;
                constexpr int RL = T::STAGES == 3 ? T::DSR : 0;
                constexpr int R1 = 2 < T::STEPS ? T::DSR : RL;
                constexpr int VM0 = LOAD_STEP == 0 ? VMR : 0;
                if (t == 0) {
                    interleave<T::MF, R0, T::DSW, VM0>();
                } else if (t == LOAD_STEP) {
                    interleave<T::MF, R1, 0, VMR>();
                } else if (t + 1 < T::STEPS) {
                    interleave<T::MF, T::DSR, 0, 0>();
                } else {
                    interleave<T::MF, RL, 0, 0>();
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
            cur = next;
        }
    };
    if (cols_inside) {
        steady(std::false_type{});
    } else {
        steady(std::true_type{});
    }

    // Remaining windows (the last STAGES ones and a partial last window): the
    // same schedule with the copies guarded.
    for (; w < w_end; ++w) {
        const float *s = lds + cur * T::STAGE;
        const int next = cur + 1 == T::STAGES ? 0 : cur + 1;
        if constexpr (T::STAGES == 2) read_frag(frag[0], s, 0);
#pragma unroll
        for (int t = 0; t < T::STEPS; ++t) {
            // Issue the reads of the following step before this step's MFMAs.  After
            // the last window the cross-window read fetches an unused stage; keeping
            // it unconditional lets the LDS wait counts stay exact.
            if (t + 1 < T::STEPS) {
                read_frag(frag[(t + 1) & 1], s, t + 1);
            } else if constexpr (T::STAGES == 3) {
                read_frag(frag[(t + 1) & 1], lds + next * T::STAGE, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            multiply(frag[t & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Window w + STAGES - 1 goes from registers to the stage freed by window w - 1,
        // and the loads of the window after it are issued.
        if (w + T::STAGES - 1 < w_end) {
            const int fill = cur == 0 ? T::STAGES - 1 : cur - 1;
            stash(fill);
            if (w + T::STAGES < w_end) fetch((w + T::STAGES) * T::BK);
        }
        __syncthreads();
        cur = next;
    }
}

// Store the accumulators of block (m0, n0) to C; rows >= M and columns >= N are
// skipped.  Accumulator r of block (i, j) holds row 8*(r/4) + 4*lh + r%4 of the
// block and column TN*lr + j of the wave's strip.
template <class T>
__device__ __forceinline__ void store_tile(const GemmArgs &g, int m0, int n0, const Acc<T> &acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int sw = wave % T::SPATIAL;
    const int wm = sw / T::WAVES_N, wn = sw % T::WAVES_N;
    const int M = g.M, N = g.N;
    float *__restrict__ C = g.C;
    const int64_t ldc = g.ldc;
    const bool full = (m0 + T::BM <= M) && (n0 + T::BN <= N);
    const int col0 = n0 + wn * T::WN + T::TN * lr;
    const int row0 = m0 + wm * T::WM + 4 * lh;
    if (full) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + i * 32 + 8 * (r >> 2) + (r & 3);
                float v[T::TN];
#pragma unroll
                for (int j = 0; j < T::TN; ++j) v[j] = acc[i][j][r];
                __builtin_memcpy(C + (int64_t)row * ldc + col0, v, sizeof(v));
            }
            // one row block at a time keeps few accumulators in flight
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + i * 32 + 8 * (r >> 2) + (r & 3);
                if (row < M) {
                    float *dst = C + (int64_t)row * ldc + col0;
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
                        if (col0 + j < N) dst[j] = acc[i][j][r];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Split-k inside the work-group: groups 1..KW-1 hand their partial blocks to
// group 0 through LDS, which adds them in group order.  Returns true for the
// waves that hold the finished block.
template <class T>
__device__ __forceinline__ bool kw_reduce(float *lds, Acc<T> &acc) {
    if constexpr (T::KW == 1) {
        return true;
    } else {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int kg = wave / T::SPATIAL, sw = wave % T::SPATIAL;
        float *red = lds + sw * 64 * T::ACC + lane;
        constexpr int GROUP_STRIDE = T::SPATIAL * 64 * T::ACC;
        if (kg > 0) {
            float *dst = red + (kg - 1) * GROUP_STRIDE;
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dst[((i * T::TN + j) * 16 + r) * 64] = acc[i][j][r];
        }
        __syncthreads();
        if (kg > 0) return false;
#pragma unroll
        for (int gi = 1; gi < T::KW; ++gi) {
            const float *src = red + (gi - 1) * GROUP_STRIDE;
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] += src[((i * T::TN + j) * 16 + r) * 64];
        }
        return true;
    }
}

template <class T>
__device__ __forceinline__ void zero_acc(Acc<T> &acc) {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = f32x16{};
}

// Data-parallel form: one work-group per BM x BN block of C.
template <class T>
__global__ __launch_bounds__(T::THREADS, T::OCC) void mfma_kernel(GemmArgs g, int tiles_m,
                                                                 int tiles_n) {
    __shared__ __attribute__((aligned(16))) float lds[T::LDS_FLOATS];
    int tm, tn;
    tile_order(blockIdx.x, tiles_m, tiles_n, T::GROUP_M, &tm, &tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    Acc<T> acc;
    zero_acc<T>(acc);
    mma_tile<T>(g, lds, m0, n0, 0, (g.K + T::BK - 1) / T::BK, acc);
    if (!kw_reduce<T>(lds, acc)) return;
    store_tile<T>(g, m0, n0, acc);
}

template <class T>
static hipError_t launch_tile(const Problem &p, hipStream_t s) {
    const int64_t tiles_m = (p.M + T::BM - 1) / T::BM;
    const int64_t tiles_n = (p.N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > INT32_MAX) return hipErrorInvalidValue;
    const GemmArgs g{p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc};
    return launch(mfma_kernel<T>, dim3((unsigned)(tiles_m * tiles_n)), dim3(T::THREADS), 0, s, g,
                  (int)tiles_m, (int)tiles_n);
}

// ---------------------------------------------------------------------------
// Tile choice.  A launch of T tiles on U compute units finishes when the busiest
// CU has worked through R = ceil(T / U) tiles, so a configuration's time is
// modelled as R * (2*BM*BN*K / (e / 256) + t1) + t0, where e is a whole-chip
// throughput in TFLOP/s, t1 a fixed cost per tile (prologue, epilogue) and t0 a
// fixed cost per launch.  Each configuration has two throughputs: one for
// products whose A and B together fit in 200 MB (inside the 256 MB Infinity
// Cache), one for larger products.  The four numbers per configuration were
// fitted (least squares on log time) to timings of every configuration on 14
// shapes on MI355X, among them the 512^3, 1024^3, 2048 x 3072 x 4096,
// 4095 x 4097 x 1023 and 8192^3 products; on 12 of them the model picks the
// fastest configuration and on the other two one within 3% of it.  The smallest
// estimate wins.
struct TileChoice {
    hipError_t (*launch)(const Problem &, hipStream_t);
    const char *name;  // block, k window, wave block, wave groups, LDS stages
    int bm, bn;
    double tflops_cached;  // e, A and B within 200 MB
    double tflops_large;   // e, larger A and B
    double t0_us;          // t0
    double t1_us;          // t1
};

// 256 x 256 blocks, one wave per SIMD with 128 x 128 of C each: large products.
using TileHuge = MfmaTile<256, 256, 16, 128, 128, 1, 8, 3>;
using TileWide = MfmaTile<128, 128, 16, 32, 128, 1, 8, 3>;
// 128 x 192 blocks of 64 x 96 per wave, k split over two wave groups (two waves
// per SIMD): one block per CU on grids of about 256 blocks, such as 2048 x 3072.
using TileSplit192 = MfmaTile<128, 192, 32, 64, 96, 2, 8, 3>;
// 192 x 128 blocks of 96 x 64 per wave.
using TileTall = MfmaTile<192, 128, 16, 96, 64, 1, 8, 3>;
using TileSmall = MfmaTile<64, 64, 16, 32, 32, 1, 4, 3>;
using TileSplit64 = MfmaTile<64, 64, 32, 32, 32, 2, 4, 3>;
// k split four ways: one 8-wide step per group and window, so two stages.
using TileTiny = MfmaTile<32, 32, 32, 32, 32, 4, 4, 2>;

static const TileChoice kTiles[] = {
    {launch_tile<TileHuge>, "256x256x16 w128x128 k1 s3", 256, 256, 148.5, 150.0, 4.0, 15.0},
    {launch_tile<TileWide>, "128x128x16 w32x128 k1 s3", 128, 128, 136.5, 137.5, 6.0, 2.0},
    {launch_tile<TileSplit192>, "128x192x32 w64x96 k2 s3", 128, 192, 138.5, 138.5, 5.0, 9.0},
    {launch_tile<TileTall>, "192x128x16 w96x64 k1 s3", 192, 128, 138.5, 143.0, 7.0, 3.0},
    {launch_tile<TileSmall>, "64x64x16 w32x32 k1 s3", 64, 64, 128.0, 122.5, 8.0, 1.0},
    {launch_tile<TileSplit64>, "64x64x32 w32x32 k2 s3", 64, 64, 125.0, 129.5, 6.0, 1.0},
    {launch_tile<TileTiny>, "32x32x32 w32x32 k4 s2", 32, 32, 101.0, 106.0, 7.0, 0.0},
};
constexpr int kTileCount = (int)(sizeof(kTiles) / sizeof(kTiles[0]));

static int compute_units() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    return cus;
}

// Index into kTiles of the configuration the model prefers for this shape.
static int choose_tile(int M, int N, int K, int cus) {
    int best = 0;
    double best_us = 0;
    for (int i = 0; i < kTileCount; ++i) {
        const TileChoice &c = kTiles[i];
        const double tiles = (double)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        const double per_cu = std::ceil(tiles / cus);
        const double operands = 4.0 * ((double)M * K + (double)K * N);
        const double per_cu_tflops =
            (operands <= 200e6 ? c.tflops_cached : c.tflops_large) / 256.0;  // fitted on 256 CUs
        const double us =
            per_cu * (2.0 * c.bm * c.bn * (double)K / (per_cu_tflops * 1e6) + c.t1_us) + c.t0_us;
        if (i == 0 || us < best_us) {
            best = i;
            best_us = us;
        }
    }
    return best;
}

hipError_t launch_mfma(const Problem &p, hipStream_t s) {
    return kTiles[choose_tile(p.M, p.N, p.K, compute_units())].launch(p, s);
}

int mfma_tile_count() { return kTileCount; }

const char *mfma_tile_name(int tile) {
    return tile >= 0 && tile < kTileCount ? kTiles[tile].name : nullptr;
}

int mfma_select(int M, int N, int K, int cus) { return choose_tile(M, N, K, cus > 0 ? cus : 256); }

hipError_t launch_mfma_tile(const Problem &p, hipStream_t s, int tile) {
    if (tile < 0 || tile >= kTileCount) return hipErrorInvalidValue;
    return kTiles[tile].launch(p, s);
}

}  // namespace sgemm
