// mfma_kernel.h -- register-blocked fp32 matrix-core kernel of the ladder, for
// either storage order of each operand.
//
// Same decomposition as the pages' tiled kernel (page "CUDA算子优化(4)：矩阵乘法",
// section "版本V1共享内存分块": each work-group owns a TILE_M x TILE_N block of C and
// slides a TILE_K window along k, staging the A and B windows in on-chip memory),
// re-sized for gfx950:
//   * a BM x BN block of C per work-group, BK-wide k windows in a ring of two or
//     three LDS stages (later windows are written while the current one is read,
//     so one barrier per window replaces the pages' two);
//   * global -> LDS copies as 16-byte loads, issued a window ahead into
//     registers so that their latency overlaps a whole window of math; when
//     every lane's offset inside a block fits 32 bits (all but rows of more
//     than about 2M floats), they are buffer loads whose base address is
//     uniform (SGPRs, advanced once per window) and whose per-lane offsets
//     stay fixed, so no vector instruction is spent on addresses;
//   * the operand fragments of the next 8-wide k step are read from LDS while
//     the MFMAs of the current step run; with three stages this reaches across
//     the window boundary, so the barrier does not leave the matrix cores idle;
//   * LDS holds the stages of A, then those of B; the steady loop runs groups
//     of STAGES windows whose stages are compile-time constants, so each LDS
//     access is one register per operand plus an immediate offset and the loop
//     issues no vector instructions for addresses (a vector instruction between
//     MFMAs costs the matrix core several cycles);
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
// Operand storage.  op(A) is M x K and op(B) is K x N.  An operand is either
// k-contiguous (A as given, or B transposed: rows of op(A), columns of op(B)
// run along memory) or mn-contiguous (A transposed, or B as given).  Its window
// is kept in LDS in the same orientation: a k-contiguous window as rows of BK
// floats (pitch BK + PAD_A), an mn-contiguous one as BK rows of BM or BN floats
// (pitch + PAD_B).  Both pitches keep the fragment reads below free of LDS bank
// conflicts (64 banks; a 16-byte read serves 16 lanes per cycle).
//
// Operand placement.  The k order inside one MFMA is fixed by the hardware.
// Across the four MFMAs of an 8-wide k step, lane half h supplies
// k = k8 + 4h + q to the q-th instruction.
//   * k-contiguous operand: a lane fetches the four consecutive k of its row
//     (column) with one 16-byte LDS read per 32-wide accumulator block; MFMA row
//     (column) r of block i is row (column) 32*i + r of the wave's strip.
//   * mn-contiguous operand: MFMA row (column) r of block i stands for row
//     (column) T*r + i of the wave's strip, T = WM/32 (WN/32), so a lane fetches
//     its T adjacent rows (columns) for one k with one LDS access, and stores of
//     C cover T adjacent columns at once.
// A and B use the same k assignment, so every product opA[i][k]*opB[k][j] is
// formed exactly once.
//
// Edges: rows and columns beyond M and N are read from the last valid one (they
// only feed outputs that are not stored); the last, partial k window is
// zero-filled on both operands (the pages' zero-fill of partial tiles), so no
// value outside the logical matrices enters a stored result and no load leaves
// the matrices' extents.
#pragma once

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

// LDS accesses needed to read N adjacent floats of one row.
constexpr int lds_reads(int n) { return n == 3 ? 2 : 1; }

// 16-byte load from a 4-byte aligned address (gfx950 global memory instructions
// accept dword-aligned multi-dword accesses).
__device__ __forceinline__ f32x4 load16(const float *p) {
    f32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// 16-byte load at byte offset `off` from the uniform address `base`, through a
// buffer resource (no range limit; the caller keeps every access inside its
// matrix).
__device__ __forceinline__ f32x4 load16_at(const char *base, uint32_t off) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, -1, 0x00020000);
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 12-byte loads into the first three lanes of a vector whose fourth is left
// undefined (it is never used): from a 4-byte aligned address, and through a
// buffer resource as load16_at.
typedef float f32x3 __attribute__((ext_vector_type(3)));

__device__ __forceinline__ f32x4 load12(const float *p) {
    f32x3 x;
    __builtin_memcpy(&x, p, 12);
    return __builtin_shufflevector(x, x, 0, 1, 2, -1);
}

__device__ __forceinline__ f32x4 load12_at(const char *base, uint32_t off) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, -1, 0x00020000);
    const f32x3 x = __builtin_bit_cast(f32x3, __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0));
    return __builtin_shufflevector(x, x, 0, 1, 2, -1);
}

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

// BM x BN block of C per work-group, BK-wide k windows, WM x WN block per wave,
// KW wave groups splitting k, GROUP_M tile-rows per ordering group, STAGES LDS
// buffers (2 or 3), OCC the number of waves per SIMD that the register
// allocation must allow, PAD_A / PAD_B the LDS row padding of k-contiguous and
// mn-contiguous windows, RING the register sets that carry windows from global
// memory to LDS (a window's loads are issued RING windows before it is stored).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int KW_, int GROUP_M_, int STAGES_ = 2,
          int OCC_ = 1, int PAD_A_ = 4, int PAD_B_ = 8, int RING_ = 1>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, KW = KW_;
    static constexpr int GROUP_M = GROUP_M_, STAGES = STAGES_, OCC = OCC_, RING = RING_;
    static constexpr int PAD_A = PAD_A_, PAD_B = PAD_B_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int SPATIAL = WAVES_M * WAVES_N;    // waves per k group
    static constexpr int THREADS = SPATIAL * KW * 64;
    static constexpr int TM = WM / 32, TN = WN / 32;     // 32x32 accumulators per wave
    static constexpr int ACC = TM * TN * 16;             // accumulator floats per lane
    static constexpr int RED = (KW - 1) * SPATIAL * 64 * ACC;  // split-k partials
    static constexpr int STEPS = BK / (8 * KW);          // 8-wide k steps per group per window
    static constexpr int MF = 4 * TM * TN;               // MFMAs per step
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "wave tiling");
    static_assert(TM >= 1 && TM <= 4 && TN >= 1 && TN <= 4,
                  "a lane holds 1 to 4 adjacent rows or columns");
    static_assert(BK % (8 * KW) == 0 && BK % 4 == 0, "k window splits into 8-wide steps");
    static_assert(BM % 4 == 0 && BN % 4 == 0, "16-byte vectors along m and n");
    static_assert(THREADS <= 1024, "work-group size");
    static_assert(PAD_A_ % 4 == 0 && PAD_B_ % 4 == 0, "16-byte aligned LDS rows");
    static_assert(STAGES == 2 || (STAGES == 3 && STEPS % 2 == 0),
                  "a three-stage ring carries fragments across windows in an even step count");
    static_assert(RING >= 1 && RING <= 4, "one to four register sets");
};

// A tile configuration with the storage order of each operand: TA (op(A) is the
// transpose of the stored K x M array) and TB (op(B) is the transpose of the
// stored N x K array); NARROW: every per-lane byte offset inside a block window
// fits 32 bits (checked on the host by narrow_offsets()); RING: the register sets
// of this instantiation (the tile's RING, or 1, chosen per launch by use_ring()).
template <class T, bool TA_, bool TB_, bool NARROW_ = true, int RING_ = T::RING>
struct Cfg : T {
    static constexpr bool TA = TA_, TB = TB_, NARROW = NARROW_;
    static constexpr int RING = RING_;  // register sets used by this instantiation
    // B as given whose lanes hold three adjacent columns (96-wide wave blocks).
    // With A as given it is copied in 12-byte pieces, one per lane's three
    // columns, each into a 16-byte slot of its LDS row (the fourth float is
    // undefined and never read into an MFMA), so a fragment is one aligned 16-byte
    // read instead of an 8-byte and a 4-byte one (B3; 2048 x 3072 x 4096: 142.1 ->
    // 143.6 TFLOP/s).  With A transposed it is loaded as 16-byte pieces of its
    // rows and written to LDS along k, as a transposed B is (BX): three 16-byte
    // fragment reads per step instead of four (365.1 -> 360.0 us at 2048 x 3072 x
    // 4096; with A as given the two forms measured within 0.2%).  The fragments
    // and the stores of C follow B's LDS layout (BKC).  The 12-byte form for A
    // transposed with 96-high wave blocks measured 1.2-1.4% slower on the 192 x
    // 128 block, so A keeps 16-byte copies.
    static constexpr bool B3 = !TA && !TB && T::TN == 3;
    static constexpr bool BX = TA && !TB && T::TN == 3;
    static constexpr bool BKC = TB || BX;  // B's LDS window: k-contiguous rows per column
    static constexpr int AW = 4, BW = B3 ? 3 : 4;           // floats per copied vector
    static constexpr int B_ROW = B3 ? T::BN / 3 * 4 : T::BN;  // LDS floats per B row
    static constexpr int PA = TA ? T::BM + T::PAD_B : T::BK + T::PAD_A;  // A window pitch
    static constexpr int PB = BKC ? T::BK + T::PAD_A : B_ROW + T::PAD_B;  // B window pitch
    static constexpr int A_STAGE = (TA ? T::BK : T::BM) * PA;
    static constexpr int B_STAGE = (BKC ? T::BN : T::BK) * PB;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_FLOATS = T::STAGES * STAGE > T::RED ? T::STAGES * STAGE : T::RED;
    // Copied vectors per window and per work-item.
    static constexpr int A_TOTAL = T::BM * T::BK / AW, B_TOTAL = T::BK * T::BN / BW;
    static constexpr int A_VECS = (A_TOTAL + T::THREADS - 1) / T::THREADS;
    static constexpr int B_VECS = (B_TOTAL + T::THREADS - 1) / T::THREADS;
    static constexpr int DSW = A_VECS + (BX ? 4 : 1) * B_VECS;  // LDS writes per window
    static constexpr int VMR = A_VECS + B_VECS;  // global loads per window
    static constexpr int DSR_A = TA ? 4 * lds_reads(T::TM) : T::TM;  // LDS reads per step
    static constexpr int DSR_B = BKC ? T::TN : 4 * (B3 ? 1 : lds_reads(T::TN));
    static constexpr int DSR = DSR_A + DSR_B;
    // The steady-state loop writes LDS in the first step of a window and issues
    // the `vmr` global loads of a later window in the same step, or in the second
    // step when one step has too few MFMAs to cover all of those memory
    // instructions.
    static constexpr int load_step(int vmr) {
        return (T::STEPS > 1 && T::MF < DSR + DSW + vmr) ? 1 : 0;
    }
    // The 128 x 128 wave blocks (one wave per SIMD, two steps per window) with A
    // as given issue the loads of A (64-byte row pieces, 16 rows per instruction)
    // in the first step, with the LDS stores, and those of B in the second,
    // instead of all of them in the first: 4095 x 4097 x 1023 263.9 -> 257.1 us,
    // 8192^3 (B as given or transposed) and 4096^3 0.3-0.4% faster.  With A
    // transposed the split was neutral to 0.5% slower, on the 128 x 128 block
    // (four 32 x 128 waves) 0.7-0.8% slower at 16384 x 16384 x 1024 and 6000 x
    // 6000 x 1000, on the 128 x 192 block 0.5% slower at 2048 x 3072 x 4096, and
    // on the 192 x 128 block neutral.
    static constexpr bool SPLIT_LOADS = T::STEPS == 2 && T::TM == 4 && T::TN == 4 && !TA;
    // The steady loop of interior blocks runs in groups of STAGES windows whose
    // LDS stages are compile-time constants, so every LDS address is a register
    // plus an immediate and the loop issues no address arithmetic (8192^3 151.1
    // -> 153.7, 2048 x 3072 x 4096 146.0 -> 149.4 TFLOP/s).  The 192 x 128 block
    // (96-high wave blocks, two work-groups per CU) measured 6-22% slower that way
    // on products 4096 wide (4096 x 4096 x 1024: 271 -> 316 us; 6000 x 6000 x 1000
    // 1% faster) and keeps one loop over run-time stages.
    static constexpr bool UNROLL_STAGES = T::TM != 3;
    static_assert(!B3 || T::BN % 3 == 0, "three-wide B rows");
    static_assert(!BX || (T::BK % 16 == 0 && T::BN % 16 == 0 && B_TOTAL % 64 == 0),
                  "B written along k: 16 rows by 4 vectors per wave");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");
};

// The operands of one product C = alpha*op(A)*op(B) + beta*C.
struct GemmArgs {
    int M, N, K;
    const float *__restrict__ A;
    int64_t lda;
    const float *__restrict__ B;
    int64_t ldb;
    float *__restrict__ C;
    int64_t ldc;
    float alpha, beta;
};

template <class T>
using Acc = f32x16[T::TM][T::TN];

// Global -> register -> LDS copy of one operand's k window, for the `VECS`
// vectors of W floats this work-item owns (vector v exists iff tid + v*THREADS <
// TOTAL; a missing one re-reads the last vector and is not stored).  Each vector
// lands in a 16-byte slot of LDS (W = 3: the fourth float is undefined and is
// never read into an MFMA).
//   k-contiguous (KC, W = 4): ROWS rows (of op(A) or columns of op(B)) of BK
//     floats; rows beyond `extent` read the last valid one.
//   mn-contiguous (W = 4 or 3): BK rows of COLS floats (along m or n); columns
//     beyond `extent` read the last valid one.
template <class T, bool KC, int ROWS_OR_COLS, int TOTAL, int VECS, int W = 4, bool XP = false>
struct Operand {
    static_assert(W == 4 || (W == 3 && !KC), "three-float vectors along m or n only");
    static constexpr int Q = KC ? T::BK / 4 : ROWS_OR_COLS / W;  // vectors per LDS row
    const float *src[VECS];  // start of the vector in window 0 (when !NARROW)
    const char *org;         // uniform: the block's first row (KC) or column
    uint32_t off[VECS];      // byte offset of src[v] from org (when NARROW)
    int lds[VECS];
    int kofs[VECS];  // KC: k offset of the vector in the window; else its k row
    int pos[VECS];   // mn-contiguous: first column (m or n) of the vector
    int pitch_;      // LDS pitch (XP: between columns)
    f32x4 r[VECS];

    __device__ __forceinline__ static bool has(int tid, int v) {
        return (TOTAL % T::THREADS == 0) || tid + v * T::THREADS < TOTAL;
    }

    // Every work-item owns every one of its vectors and vector v lies THREADS/Q
    // rows after vector 0 (both placements below keep q and add THREADS/Q to the
    // row): its LDS slot is a fixed distance after vector 0's, so a window's
    // stores need one address and immediate offsets.
    static constexpr bool LINEAR = !XP && TOTAL % T::THREADS == 0 && T::THREADS % Q == 0;

    // Vector c of the window -> its row and its vector q within the row.  A
    // k-contiguous window of four vectors per row (16-wide k windows, rows padded
    // to 20 floats) hands the 16 rows of each 64-vector chunk out so that every 16
    // consecutive work-items store rows r, r+4, r+8 and r+12: at a pitch of 20
    // floats those rows start 16 banks apart and together fill the 64 banks once,
    // where rows r..r+3 would wrap onto the same banks (a two-way conflict on the
    // 16-byte LDS stores).  Each work-item still loads a whole 16-byte vector and
    // each wave the same 64-byte row pieces.
    __device__ __forceinline__ static void place(int c, int &row, int &q) {
        if constexpr (XP) {
            // mn-contiguous window written along k: each wave loads 16 rows by 4
            // vectors (64 bytes of each row); its 4-byte LDS stores of one column
            // offset e then land in 64 different banks (pitch BK + 4 = 36 floats)
            const int l = c & 63, chunk = c >> 6;
            constexpr int KB = T::BK / 16;
            row = 16 * (chunk % KB) + (l >> 2);
            q = 4 * (chunk / KB) + (l & 3);
        } else if constexpr (KC && Q == 4 && TOTAL % 64 == 0 && T::BK + T::PAD_A == 20) {
            const int l = c & 63;
            row = (c >> 6) * 16 + ((l >> 2) & 3) * 4 + (l >> 4);
            q = l & 3;
        } else {
            row = c / Q;
            q = c % Q;
        }
    }

    // origin: first row (KC) or column of the block; extent: M or N; ld: row
    // stride of the stored array; base/pitch: LDS placement of the window.
    __device__ __forceinline__ void init(const float *X, int64_t ld, int origin, int extent,
                                         int base, int pitch, int tid) {
#pragma unroll
        for (int v = 0; v < VECS; ++v) {
            const int c = min(tid + v * T::THREADS, TOTAL - 1);
            int row, q;
            place(c, row, q);
            if constexpr (KC) {
                const int gr = min(origin + row, extent - 1);
                src[v] = X + (int64_t)gr * ld + q * 4;
                org = (const char *)(X + (int64_t)origin * ld);
                off[v] = (uint32_t)(((int64_t)(gr - origin) * ld + q * 4) * 4);
                kofs[v] = q * 4;
                pos[v] = 0;
            } else {
                src[v] = X + (int64_t)row * ld + origin + q * W;
                org = (const char *)(X + origin);
                off[v] = (uint32_t)(((int64_t)row * ld + q * W) * 4);
                kofs[v] = row;
                pos[v] = origin + q * W;
            }
            // XP: column q*W + e of the window at k = row, in rows of BK per column
            lds[v] = XP ? base + q * W * pitch + row : base + row * pitch + q * 4;
        }
        pitch_ = pitch;
    }

    // Start of vector v in window 0.
    __device__ __forceinline__ const float *at(int v) const {
        if constexpr (T::NARROW) {
            return (const float *)(org + off[v]);
        } else {
            return src[v];
        }
    }

    // W floats of row `row` (an mn row of the window) from column pos[v] on, each
    // index clamped to extent - 1.
    __device__ __forceinline__ f32x4 clamped(const float *row, int v, int extent) const {
        f32x4 x;
        x.x = row[min(pos[v] + 0, extent - 1)];
        x.y = row[min(pos[v] + 1, extent - 1)];
        x.z = row[min(pos[v] + 2, extent - 1)];
        x.w = W == 4 ? row[min(pos[v] + 3, extent - 1)] : 0.0f;
        return x;
    }

    // Full window at k0 (every k < K).  INSIDE: every column of an mn-contiguous
    // block lies inside its matrix, so whole vectors are read.
    template <bool INSIDE>
    __device__ __forceinline__ void fetch_full(int64_t k0, int64_t ld, int extent) {
#pragma unroll
        for (int v = 0; v < VECS; ++v) {
            if constexpr (KC && T::NARROW) {
                r[v] = load16_at(org + k0 * 4, off[v]);
            } else if constexpr (KC) {
                r[v] = load16(src[v] + k0);
            } else if constexpr (INSIDE && T::NARROW) {
                r[v] = W == 4 ? load16_at(org + k0 * ld * 4, off[v])
                              : load12_at(org + k0 * ld * 4, off[v]);
            } else if constexpr (INSIDE) {
                r[v] = W == 4 ? load16(src[v] + k0 * ld) : load12(src[v] + k0 * ld);
            } else {
                r[v] = clamped(at(v) + k0 * ld - pos[v], v, extent);
            }
        }
    }

    // Any window: the general form of fetch_full, zeroing every element with k >= K.
    __device__ __forceinline__ void fetch(int64_t k0, int64_t ld, int extent, int K,
                                          bool inside) {
        if (k0 + T::BK <= K) {
            if (inside) {
                fetch_full<true>(k0, ld, extent);
            } else {
                fetch_full<false>(k0, ld, extent);
            }
            return;
        }
#pragma unroll
        for (int v = 0; v < VECS; ++v) {
            if constexpr (KC) {
                const int64_t kv = K - (k0 + kofs[v]);
                const float *p = at(v) + k0;
                r[v].x = kv > 0 ? p[0] : 0.0f;
                r[v].y = kv > 1 ? p[1] : 0.0f;
                r[v].z = kv > 2 ? p[2] : 0.0f;
                r[v].w = kv > 3 ? p[3] : 0.0f;
            } else {
                if (k0 + kofs[v] < K) {
                    r[v] = clamped(at(v) + k0 * ld - pos[v], v, extent);
                } else {
                    r[v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
        }
    }

    __device__ __forceinline__ void stash(float *stage, int tid) const {
#pragma unroll
        for (int v = 0; v < VECS; ++v)
            if (has(tid, v)) {
                const int at = LINEAR ? lds[0] + v * (T::THREADS / Q) * pitch_ : lds[v];
                if constexpr (XP) {
                    stage[lds[v]] = r[v].x;
                    stage[lds[v] + pitch_] = r[v].y;
                    stage[lds[v] + 2 * pitch_] = r[v].z;
                    stage[lds[v] + 3 * pitch_] = r[v].w;
                } else if constexpr (W == 3) {
                    // the first three floats of the 16-byte slot (one 12-byte store)
                    typedef float f32x3s __attribute__((ext_vector_type(3), aligned(16)));
                    *(f32x3s *)(stage + at) = f32x3s{r[v].x, r[v].y, r[v].z};
                } else {
                    *(f32x4 *)(stage + at) = r[v];
                }
            }
    }
};

// acc += the product of op(A) rows m0..m0+BM-1 and op(B) columns n0..n0+BN-1
// over the k windows [w_begin, w_end) (window w covers k = w*BK .. w*BK+BK-1).
// Called by every work-item of the group; uses all of `lds` and ends on a
// barrier, so LDS is free again when it returns.
template <class C>
__device__ __forceinline__ void mma_tile(const GemmArgs &g, float *lds, int m0, int n0,
                                         int w_begin, int w_end, Acc<C> &acc) {
    // mn-contiguous fragments: the lane's TM (TN) adjacent values of one k; with
    // B3 the three values of B sit in a 16-byte slot.
    typedef typename VecOf<C::TM>::type AVec;
    typedef typename std::conditional<C::B3, f32x4, typename VecOf<C::TN>::type>::type BVec;
    constexpr int BL = C::B3 ? 4 : C::TN;  // lane_of width of B fragments
    const int M = g.M, N = g.N, K = g.K;
    const int64_t lda = g.lda, ldb = g.ldb;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int kg = wave / C::SPATIAL, sw = wave % C::SPATIAL;
    const int wm = sw / C::WAVES_N, wn = sw % C::WAVES_N;

    Operand<C, !C::TA, C::BM, C::A_TOTAL, C::A_VECS, C::AW> a;
    Operand<C, C::TB, C::BN, C::B_TOTAL, C::B_VECS, C::BW, C::BX> b;
    a.init(g.A, lda, m0, M, 0, C::PA, tid);
    b.init(g.B, ldb, n0, N, 0, C::PB, tid);
    // mn-contiguous blocks that reach past their matrix read clamped columns
    const bool a_inside = !C::TA || m0 + C::BM <= M;
    const bool b_inside = C::TB || n0 + C::BN <= N;
    const bool interior = a_inside && b_inside;

    auto fetch = [&](int64_t k0) {
        a.fetch(k0, lda, M, K, a_inside);
        b.fetch(k0, ldb, N, K, b_inside);
    };
    // LDS holds the STAGES windows of A, then the STAGES windows of B.  With a
    // stage index known at compile time every LDS address in the loop is one
    // register per operand plus an immediate offset.
    auto a_stage = [&](int stage) { return lds + stage * C::A_STAGE; };
    auto b_stage = [&](int stage) { return lds + C::STAGES * C::A_STAGE + stage * C::B_STAGE; };
    auto stash = [&](int stage) {
        a.stash(a_stage(stage), tid);
        b.stash(b_stage(stage), tid);
    };

    // Fragment placement (see the header comment).
    const int a_frag = C::TA ? (4 * lh) * C::PA + wm * C::WM + C::TM * lr
                             : (wm * C::WM + lr) * C::PA + 4 * lh;
    const int b_frag = C::BKC ? (wn * C::WN + lr) * C::PB + 4 * lh
                              : (4 * lh) * C::PB + (C::B3 ? (wn * C::WN / 3 + lr) * 4
                                                          : wn * C::WN + C::TN * lr);

    // Fragments of one 8-wide k step.
    struct Frag {
        typename std::conditional<C::TA, AVec[4], f32x4[C::TM]>::type a;
        typename std::conditional<C::BKC, f32x4[C::TN], BVec[4]>::type b;
    };
    auto read_frag = [&](Frag &f, int stage, int t) {
        const float *sa = a_stage(stage), *sb = b_stage(stage);
        const int k8 = (t * C::KW + kg) * 8;
        if constexpr (C::TA) {
#pragma unroll
            for (int q = 0; q < 4; ++q) f.a[q] = *(const AVec *)(sa + a_frag + (k8 + q) * C::PA);
        } else {
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
                f.a[i] = *(const f32x4 *)(sa + a_frag + i * 32 * C::PA + k8);
        }
        if constexpr (C::BKC) {
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                f.b[j] = *(const f32x4 *)(sb + b_frag + j * 32 * C::PB + k8);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) f.b[q] = *(const BVec *)(sb + b_frag + (k8 + q) * C::PB);
        }
    };
    auto multiply = [&](const Frag &f) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    float av, bv;
                    if constexpr (C::TA) {
                        av = lane_of<C::TM>(f.a[q], i);
                    } else {
                        av = f.a[i][q];
                    }
                    if constexpr (C::BKC) {
                        bv = f.b[j][q];
                    } else {
                        bv = lane_of<BL>(f.b[q], j);
                    }
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[i][j], 0, 0, 0);
                }
    };

    if constexpr (C::RING == 1) {
        // Prologue: the first STAGES-1 windows go to LDS, the next one to registers.
        // Every load of these windows is issued before any of them is waited for (a
        // second register set holds window w_begin + 1), so the first MFMA waits for
        // one memory round trip, not one per window.
        {
            auto a1 = a;
            auto b1 = b;
            const bool second = w_begin + 1 < w_end;
            fetch((int64_t)w_begin * C::BK);
            if (second) {
                a1.fetch((int64_t)(w_begin + 1) * C::BK, lda, M, K, a_inside);
                b1.fetch((int64_t)(w_begin + 1) * C::BK, ldb, N, K, b_inside);
            }
            stash(0);
            if constexpr (C::STAGES == 3) {
                if (w_begin + 2 < w_end) fetch((int64_t)(w_begin + 2) * C::BK);
                if (second) {
                    a1.stash(a_stage(1), tid);
                    b1.stash(b_stage(1), tid);
                }
            } else {
                if (second) {
    #pragma unroll
                    for (int v = 0; v < C::A_VECS; ++v) a.r[v] = a1.r[v];
    #pragma unroll
                    for (int v = 0; v < C::B_VECS; ++v) b.r[v] = b1.r[v];
                }
            }
        }
        __syncthreads();

        Frag frag[2];
        int cur = 0;  // LDS stage of window w
        int w = w_begin;
        if constexpr (C::STAGES == 3) read_frag(frag[0], 0, 0);

        // Steady state: a window whose successors up to w + STAGES are all full.
        // The body has no branches, so the copies of later windows (LDS stores of
        // window w + STAGES - 1, global loads of window w + STAGES) and the fragment
        // reads of the next step are spread one by one between the MFMAs instead of
        // stalling the matrix cores in a block of their own.  Work-groups whose
        // block reaches past M or N on an mn-contiguous operand (EDGE) load that
        // operand one element at a time with the index clamped, which keeps the
        // body free of branches there too.
        auto steady = [&](auto edge_tag) {
            constexpr bool EDGE = decltype(edge_tag)::value;
            constexpr int VMR = EDGE ? (C::TA ? 4 : 1) * C::A_VECS + (C::TB ? 1 : C::BW) * C::B_VECS
                                     : C::VMR;
            constexpr int LOAD_STEP = C::load_step(VMR);
            const int steady_end = min(w_end, K / C::BK) - C::STAGES;
            // Window wi in LDS stage `stage` (a compile-time constant, or an int).
            auto window = [&](auto stage, int wi) {
                const int cs = stage;
                const int next = cs + 1 == C::STAGES ? 0 : cs + 1;
                const int fill = cs == 0 ? C::STAGES - 1 : cs - 1;
                if constexpr (C::STAGES == 2) read_frag(frag[0], cs, 0);
    #pragma unroll
                for (int t = 0; t < C::STEPS; ++t) {
                    if (t + 1 < C::STEPS) {
                        read_frag(frag[(t + 1) & 1], cs, t + 1);
                    } else if constexpr (C::STAGES == 3) {
                        read_frag(frag[(t + 1) & 1], next, 0);
                    }
                    if (t == 0) stash(fill);
                    if constexpr (C::SPLIT_LOADS) {
                        const int64_t k0 = (int64_t)(wi + C::STAGES) * C::BK;
                        if (t == 0) a.template fetch_full<!EDGE>(k0, lda, M);
                        if (t == 1) b.template fetch_full<!EDGE>(k0, ldb, N);
                    } else if (t == LOAD_STEP) {
                        const int64_t k0 = (int64_t)(wi + C::STAGES) * C::BK;
                        a.template fetch_full<!EDGE>(k0, lda, M);
                        b.template fetch_full<!EDGE>(k0, ldb, N);
                    }
                    multiply(frag[t & 1]);
                    // LDS reads issued in step 0, in a middle step and in the last step.
                    constexpr int R0 = (1 < C::STEPS || C::STAGES == 3) ? C::DSR : 0;
                    constexpr int RL = C::STAGES == 3 ? C::DSR : 0;
                    constexpr int R1 = 2 < C::STEPS ? C::DSR : RL;
                    constexpr int VM0 = LOAD_STEP == 0 ? VMR : 0;
                    constexpr int VMA = EDGE ? (C::TA ? 4 : 1) * C::A_VECS : C::A_VECS;
                    constexpr int VMB = VMR - VMA;
                    if (C::SPLIT_LOADS && t == 0) {
                        interleave<C::MF, R0, C::DSW, VMA>();
                    } else if (C::SPLIT_LOADS) {
                        interleave<C::MF, RL, 0, VMB>();
                    } else if (t == 0) {
                        interleave<C::MF, R0, C::DSW, VM0>();
                    } else if (t == LOAD_STEP) {
                        interleave<C::MF, R1, 0, VMR>();
                    } else if (t + 1 < C::STEPS) {
                        interleave<C::MF, C::DSR, 0, 0>();
                    } else {
                        interleave<C::MF, RL, 0, 0>();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                __syncthreads();
            };
            // Groups of STAGES windows begin and end in stage 0, so the stage of
            // every window in them is a constant (interior blocks; edge blocks
            // keep the loop below, whose clamped loads need more registers).
            if constexpr (C::UNROLL_STAGES && !EDGE) {
                if (cur == 0) {
                    for (; w + C::STAGES <= steady_end; w += C::STAGES) {
                        window(std::integral_constant<int, 0>{}, w);
                        window(std::integral_constant<int, 1>{}, w + 1);
                        if constexpr (C::STAGES == 3)
                            window(std::integral_constant<int, 2>{}, w + 2);
                    }
                }
            }
            for (; w < steady_end; ++w) {
                window(cur, w);
                cur = cur + 1 == C::STAGES ? 0 : cur + 1;
            }
        };
        if (interior) {
            steady(std::false_type{});
        } else {
            steady(std::true_type{});
        }

        // Remaining windows (the last STAGES ones and a partial last window): the
        // same schedule with the copies guarded.
        for (; w < w_end; ++w) {
            const int next = cur + 1 == C::STAGES ? 0 : cur + 1;
            if constexpr (C::STAGES == 2) read_frag(frag[0], cur, 0);
    #pragma unroll
            for (int t = 0; t < C::STEPS; ++t) {
                // Issue the reads of the following step before this step's MFMAs.  After
                // the last window the cross-window read fetches an unused stage; keeping
                // it unconditional lets the LDS wait counts stay exact.
                if (t + 1 < C::STEPS) {
                    read_frag(frag[(t + 1) & 1], cur, t + 1);
                } else if constexpr (C::STAGES == 3) {
                    read_frag(frag[(t + 1) & 1], next, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                multiply(frag[t & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Window w + STAGES - 1 goes from registers to the stage freed by window w - 1,
            // and the loads of the window after it are issued.
            if (w + C::STAGES - 1 < w_end) {
                const int fill = cur == 0 ? C::STAGES - 1 : cur - 1;
                stash(fill);
                if (w + C::STAGES < w_end) fetch((int64_t)(w + C::STAGES) * C::BK);
            }
            __syncthreads();
            cur = next;
        }
    } else {
        // Register ring.  Window i (counted from w_begin) is carried from its loads
        // to its LDS store by register set i % RING.  In the window that stores
        // window i + STAGES - 1 (from set Q) the loads of window i + STAGES - 1 +
        // RING go into the same set, so every window's loads have RING windows to
        // arrive instead of one.  The loop runs in groups of RING windows so that
        // each set index is a constant.
        constexpr int S = C::STAGES, R = C::RING;
        const int n = w_end - w_begin;
        decltype(a) as[R];
        decltype(b) bs[R];
#pragma unroll
        for (int q = 0; q < R; ++q) {
            as[q] = a;
            bs[q] = b;
        }
        auto win_k0 = [&](int i) { return (int64_t)(w_begin + i) * C::BK; };
        // Prologue: windows 0 .. S-2 into LDS stages 0 .. S-2 through temporaries,
        // windows S-1 .. S-2+R into their ring sets; every load issued before any
        // is waited for.
        {
            decltype(a) pa[S - 1];
            decltype(b) pb[S - 1];
#pragma unroll
            for (int j = 0; j < S - 1; ++j) {
                pa[j] = a;
                pb[j] = b;
                if (j < n) {
                    pa[j].fetch(win_k0(j), lda, M, K, a_inside);
                    pb[j].fetch(win_k0(j), ldb, N, K, b_inside);
                }
            }
#pragma unroll
            for (int u = 0; u < R; ++u) {
                if (S - 1 + u < n) {
                    as[(S - 1 + u) % R].fetch(win_k0(S - 1 + u), lda, M, K, a_inside);
                    bs[(S - 1 + u) % R].fetch(win_k0(S - 1 + u), ldb, N, K, b_inside);
                }
            }
#pragma unroll
            for (int j = 0; j < S - 1; ++j) {
                if (j < n) {
                    pa[j].stash(a_stage(j), tid);
                    pb[j].stash(b_stage(j), tid);
                }
            }
        }
        __syncthreads();

        Frag frag[2];
        int cur = 0;  // LDS stage of the current window
        if constexpr (S == 3) read_frag(frag[0], 0, 0);
        // Windows whose ring loads (window i + S - 1 + R) are full windows run the
        // branch-free schedule; the rest guard their stores and loads.
        const int steady_n = min(n, K / C::BK - w_begin) - S - R + 1;

        auto window = [&](auto q_tag, auto edge_tag, auto steady_tag, int i) {
            constexpr int Q = decltype(q_tag)::value;
            constexpr bool EDGE = decltype(edge_tag)::value;
            constexpr bool STEADY = decltype(steady_tag)::value;
            constexpr int VMR = EDGE ? (C::TA ? 4 : 1) * C::A_VECS + (C::TB ? 1 : C::BW) * C::B_VECS
                                     : C::VMR;
            constexpr int LOAD_STEP = C::load_step(VMR);
            const int next = cur + 1 == S ? 0 : cur + 1;
            const int fill = cur == 0 ? S - 1 : cur - 1;
            float *fill_a = a_stage(fill), *fill_b = b_stage(fill);
            if constexpr (S == 2) read_frag(frag[0], cur, 0);
#pragma unroll
            for (int t = 0; t < C::STEPS; ++t) {
                if (t + 1 < C::STEPS) {
                    read_frag(frag[(t + 1) & 1], cur, t + 1);
                } else if constexpr (S == 3) {
                    read_frag(frag[(t + 1) & 1], next, 0);
                }
                if constexpr (STEADY) {
                    if (t == 0) {
                        as[Q].stash(fill_a, tid);
                        bs[Q].stash(fill_b, tid);
                    }
                    if (t == LOAD_STEP) {
                        const int64_t k0 = win_k0(i + S - 1 + R);
                        as[Q].template fetch_full<!EDGE>(k0, lda, M);
                        bs[Q].template fetch_full<!EDGE>(k0, ldb, N);
                    }
                    multiply(frag[t & 1]);
                    constexpr int R0 = (1 < C::STEPS || S == 3) ? C::DSR : 0;
                    constexpr int RL = S == 3 ? C::DSR : 0;
                    constexpr int R1 = 2 < C::STEPS ? C::DSR : RL;
                    constexpr int VM0 = LOAD_STEP == 0 ? VMR : 0;
                    if (t == 0) {
                        interleave<C::MF, R0, C::DSW, VM0>();
                    } else if (t == LOAD_STEP) {
                        interleave<C::MF, R1, 0, VMR>();
                    } else if (t + 1 < C::STEPS) {
                        interleave<C::MF, C::DSR, 0, 0>();
                    } else {
                        interleave<C::MF, RL, 0, 0>();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                } else {
                    __builtin_amdgcn_sched_barrier(0);
                    multiply(frag[t & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (!STEADY) {
                if (i + S - 1 < n) {
                    as[Q].stash(fill_a, tid);
                    bs[Q].stash(fill_b, tid);
                    if (i + S - 1 + R < n) {
                        as[Q].fetch(win_k0(i + S - 1 + R), lda, M, K, a_inside);
                        bs[Q].fetch(win_k0(i + S - 1 + R), ldb, N, K, b_inside);
                    }
                }
            }
            __syncthreads();
            cur = next;
        };
        // Whole groups of R steady windows run in a loop with no branch between a
        // set's loads and its store, issuing the sets' loads in the prologue's order,
        // so each store waits only for its own set; the windows after them (fewer
        // than R that could still be steady, and the last S - 1 + R) take the
        // guarded form.
        auto run = [&](auto edge_tag) {
            int i0 = 0;
            auto group = [&](auto steady_tag) {
                auto one = [&](auto u_tag) {
                    constexpr int U = decltype(u_tag)::value;
                    if constexpr (U < R) {
                        using Qt = std::integral_constant<int, (U + S - 1) % R>;
                        if constexpr (decltype(steady_tag)::value) {
                            window(Qt{}, edge_tag, steady_tag, i0 + U);
                        } else if (i0 + U < n) {
                            window(Qt{}, edge_tag, steady_tag, i0 + U);
                        }
                    }
                };
                one(std::integral_constant<int, 0>{});
                one(std::integral_constant<int, 1>{});
                one(std::integral_constant<int, 2>{});
                one(std::integral_constant<int, 3>{});
            };
            const int steady_groups = steady_n > 0 ? steady_n / R : 0;
            for (int g = 0; g < steady_groups; ++g, i0 += R) group(std::true_type{});
            // steady windows that do not fill a whole group
            const int rest = steady_n > 0 ? steady_n - steady_groups * R : 0;
            auto rest_one = [&](auto u_tag) {
                constexpr int U = decltype(u_tag)::value;
                if constexpr (U + 1 < R) {
                    if (U < rest) {
                        using Qt = std::integral_constant<int, (U + S - 1) % R>;
                        window(Qt{}, edge_tag, std::true_type{}, i0 + U);
                    }
                }
            };
            rest_one(std::integral_constant<int, 0>{});
            rest_one(std::integral_constant<int, 1>{});
            rest_one(std::integral_constant<int, 2>{});
            // the guarded windows continue the set cycle where the steady ones stopped
            auto tail_from = [&](auto r_tag) {
                constexpr int R0 = decltype(r_tag)::value;
                for (int i = i0 + R0; i < n; i += R) {
                    auto one = [&](auto u_tag) {
                        constexpr int U = decltype(u_tag)::value;
                        if constexpr (U < R) {
                            using Qt = std::integral_constant<int, (R0 + U + S - 1) % R>;
                            if (i + U < n) window(Qt{}, edge_tag, std::false_type{}, i + U);
                        }
                    };
                    one(std::integral_constant<int, 0>{});
                    one(std::integral_constant<int, 1>{});
                    one(std::integral_constant<int, 2>{});
                    one(std::integral_constant<int, 3>{});
                }
            };
            switch (rest) {
            case 0: tail_from(std::integral_constant<int, 0>{}); break;
            case 1: if constexpr (R > 1) tail_from(std::integral_constant<int, 1>{}); break;
            case 2: if constexpr (R > 2) tail_from(std::integral_constant<int, 2>{}); break;
            default: if constexpr (R > 3) tail_from(std::integral_constant<int, 3>{}); break;
            }
        };
        if (interior) {
            run(std::false_type{});
        } else {
            run(std::true_type{});
        }
    }
}

// Store the accumulators of block (m0, n0) to C; rows outside [m_lo, M) and
// columns outside [n_lo, N) are skipped (m_lo > m0 or n_lo > n0 for a block
// moved back from the edge, whose first rows or columns belong to its
// neighbour).  Accumulator r of block (i, j) holds MFMA row rho = 8*(r/4) +
// 4*lh + r%4 and MFMA column lr of that block, placed as described in the header.
template <class C>
__device__ __forceinline__ void store_tile(const GemmArgs &g, int m0, int n0, const Acc<C> &acc,
                                           int m_lo, int n_lo, int r_first = 0, int r_count = 16) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int sw = wave % C::SPATIAL;
    const int wm = sw / C::WAVES_N, wn = sw % C::WAVES_N;
    const int M = g.M, N = g.N;
    float *__restrict__ Cm = g.C;
    const int64_t ldc = g.ldc;
    const float alpha = g.alpha, beta = g.beta;
    const bool full = (m0 + C::BM <= M) && (n0 + C::BN <= N) && m_lo == m0 && n_lo == n0;
    const int strip_m = m0 + wm * C::WM, strip_n = n0 + wn * C::WN;
    auto row_of = [&](int i, int r) {
        const int rho = 8 * (r >> 2) + 4 * lh + (r & 3);
        return strip_m + (C::TA ? C::TM * rho + i : 32 * i + rho);
    };
    // mn-contiguous B: a lane's TN adjacent columns; k-contiguous B: one column per block
    const int col0 = strip_n + (C::BKC ? lr : C::TN * lr);
    auto col_of = [&](int j) { return col0 + (C::BKC ? 32 * j : j); };
    auto put = [&](float *dst, float v) { *dst = epilogue(v, alpha, beta, dst); };
    // mn-contiguous B: the lane's TN adjacent columns of row r of block row i as one
    // access (read-modify-write when beta != 0).
    auto put_row = [&](float *dst, int i, int r) {
        float v[C::TN];
        if (beta == 0.0f) {
#pragma unroll
            for (int j = 0; j < C::TN; ++j) v[j] = alpha * acc[i][j][r];
        } else {
            float old[C::TN];
            __builtin_memcpy(old, dst + col0, sizeof(old));
#pragma unroll
            for (int j = 0; j < C::TN; ++j) v[j] = fmaf(beta, old[j], alpha * acc[i][j][r]);
        }
        __builtin_memcpy(dst + col0, v, sizeof(v));
    };
    // registers [r_first, r_first + r_count) of each block belong to this wave
    auto mine = [&](int r) { return r >= r_first && r < r_first + r_count; };
    if (full) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (!mine(r)) continue;
                float *dst = Cm + (int64_t)row_of(i, r) * ldc;
                if constexpr (!C::BKC) {
                    put_row(dst, i, r);
                } else {
#pragma unroll
                    for (int j = 0; j < C::TN; ++j) put(dst + col_of(j), acc[i][j][r]);
                }
            }
            // one row block at a time keeps few accumulators in flight
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        // Edge blocks skip rows outside [m_lo, M); a lane whose TN adjacent
        // columns all lie inside [n_lo, N) still stores them as one access (a
        // block past M only, such as the last block row of a 4095-row product,
        // then stores as fast as the others: all blocks finish together, so one
        // slow epilogue delays them all).
        const bool row_inside = !C::BKC && col0 >= n_lo && col0 + C::TN <= N;
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row_of(i, r);
                if (mine(r) && row >= m_lo && row < M) {
                    float *dst = Cm + (int64_t)row * ldc;
                    if (row_inside) {
                        if constexpr (!C::BKC) put_row(dst, i, r);
                    } else {
#pragma unroll
                        for (int j = 0; j < C::TN; ++j)
                            if (col_of(j) >= n_lo && col_of(j) < N)
                                put(dst + col_of(j), acc[i][j][r]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Split-k inside the work-group: the KW groups of waves that share a block of C
// each finish RPG = 16/KW of the 16 accumulator registers of every 32x32 block,
// group g registers [g*RPG, (g+1)*RPG).  Every wave writes the registers that the
// other groups finish to LDS (16-byte accesses, lane-contiguous), and each group
// adds the KW partials of its own registers in group order 0, 1, ..., KW-1, the
// order one group adding them all would use, so the sum is the same bit for
// bit.  All waves then store their own registers, so the reduction and the
// stores are spread over every wave of the group.  Returns the first register
// this wave stores; it stores RPG of them.
template <class C>
struct KwReduce {
    static constexpr int RPG = 16 / C::KW;                  // registers per group
    static constexpr int SLICE = C::TM * C::TN * RPG * 64;  // floats one wave hands one group
    static_assert(C::KW == 1 || RPG % 4 == 0, "whole 16-byte register runs per group");

    // Offset of register run (i, j, q) (registers 4q..4q+3 of the group's RPG) of
    // the slice that group h hands group g, for spatial wave sw and this lane.
    __device__ __forceinline__ static int at(int h, int g, int sw, int lane, int i, int j, int q) {
        const int slot = h * (C::KW - 1) + (g < h ? g : g - 1);
        return (slot * C::SPATIAL + sw) * SLICE + (((i * C::TN + j) * (RPG / 4) + q) * 64 + lane) * 4;
    }

    template <int G>
    __device__ __forceinline__ static void finish(const float *lds, Acc<C> &acc, int sw, int lane) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int q = 0; q < RPG / 4; ++q) {
                    f32x4 part[C::KW];
#pragma unroll
                    for (int h = 0; h < C::KW; ++h) {
                        if (h == G) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) part[h][e] = acc[i][j][G * RPG + 4 * q + e];
                        } else {
                            part[h] = *(const f32x4 *)(lds + at(h, G, sw, lane, i, j, q));
                        }
                    }
                    f32x4 sum = part[0];
#pragma unroll
                    for (int h = 1; h < C::KW; ++h) sum += part[h];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][G * RPG + 4 * q + e] = sum[e];
                }
    }

    __device__ __forceinline__ static int run(float *lds, Acc<C> &acc) {
        if constexpr (C::KW == 1) {
            return 0;
        } else {
            const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
            const int kg = wave / C::SPATIAL, sw = wave % C::SPATIAL;
#pragma unroll
            for (int g = 0; g < C::KW; ++g) {
                if (g == kg) continue;
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
#pragma unroll
                    for (int j = 0; j < C::TN; ++j)
#pragma unroll
                        for (int q = 0; q < RPG / 4; ++q) {
                            f32x4 v;
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][g * RPG + 4 * q + e];
                            *(f32x4 *)(lds + at(kg, g, sw, lane, i, j, q)) = v;
                        }
            }
            __syncthreads();
            switch (kg) {
            case 0: finish<0>(lds, acc, sw, lane); break;
            case 1: finish<1>(lds, acc, sw, lane); break;
            case 2: if constexpr (C::KW > 2) finish<2>(lds, acc, sw, lane); break;
            default: if constexpr (C::KW > 3) finish<3>(lds, acc, sw, lane); break;
            }
            return kg * RPG;
        }
    }
};

template <class C>
__device__ __forceinline__ void zero_acc(Acc<C> &acc) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x16{};
}

// A block that reaches past M on an m-contiguous op(A), or past N on an
// n-contiguous op(B), would have to load that operand element by element with
// clamped indices; all blocks of a launch finish together, so that one slow
// block row or column sets the time of the launch.  When the matrix holds a
// whole block in that direction, the block is moved back to end exactly at M
// (or N): it computes BM x BN outputs entirely inside C with whole 16-byte
// loads, and stores only from its original first row (column) on, the rows
// before that belonging to its neighbour.
template <class C>
__device__ __forceinline__ void edge_origin(int M, int N, int &m0, int &n0) {
    if (C::TA && m0 + C::BM > M && M >= C::BM) m0 = M - C::BM;
    if (!C::TB && n0 + C::BN > N && N >= C::BN) n0 = N - C::BN;
}

// Data-parallel form: one work-group per BM x BN block of C.
template <class C>
__global__ __launch_bounds__(C::THREADS, C::OCC) void mfma_kernel(GemmArgs g, int tiles_m,
                                                                 int tiles_n) {
    __shared__ __attribute__((aligned(16))) float lds[C::LDS_FLOATS];
    int tm, tn;
    tile_order(blockIdx.x, tiles_m, tiles_n, C::GROUP_M, &tm, &tn);
    const int m_lo = tm * C::BM, n_lo = tn * C::BN;
    int m0 = m_lo, n0 = n_lo;
    edge_origin<C>(g.M, g.N, m0, n0);
    Acc<C> acc;
    zero_acc<C>(acc);
    mma_tile<C>(g, lds, m0, n0, 0, (g.K + C::BK - 1) / C::BK, acc);
    const int r_first = KwReduce<C>::run(lds, acc);
    store_tile<C>(g, m0, n0, acc, m_lo, n_lo, r_first, KwReduce<C>::RPG);
}

// True when every per-lane byte offset from a block's first row or column
// stays below 2^31: (rows of one window - 1) * ld + one row of the window.
template <class T, bool TA, bool TB>
bool narrow_offsets(const Problem &p) {
    auto fits = [](int64_t rows, int64_t ld, int64_t row_len) {
        return ((rows - 1) * ld + row_len) * 4 < ((int64_t)1 << 31);
    };
    const bool a = TA ? fits(T::BK, p.lda, T::BM) : fits(T::BM, p.lda, T::BK);
    const bool b = TB ? fits(T::BN, p.ldb, T::BK) : fits(T::BK, p.ldb, T::BN);
    return a && b;
}

// Split-k form: work-group b computes block b % tiles over slice b / tiles of the
// k windows (slice q of S covers windows [q*W/S, (q+1)*W/S)) and stores its
// partial block, unscaled, to plane q of the workspace (M x N, row stride N).
// splitk_reduce_kernel (basic.hip) adds the planes in an order fixed by the shape.
template <class C>
__global__ __launch_bounds__(C::THREADS, C::OCC) void mfma_splitk_kernel(GemmArgs g, int tiles_m,
                                                                        int tiles_n, int slices,
                                                                        float *ws) {
    __shared__ __attribute__((aligned(16))) float lds[C::LDS_FLOATS];
    const int tiles = tiles_m * tiles_n;
    const int t = blockIdx.x % tiles, slice = blockIdx.x / tiles;
    int tm, tn;
    group_tile(t, tiles_m, tiles_n, C::GROUP_M, &tm, &tn);
    const int m_lo = tm * C::BM, n_lo = tn * C::BN;
    int m0 = m_lo, n0 = n_lo;
    edge_origin<C>(g.M, g.N, m0, n0);
    const int nwin = (g.K + C::BK - 1) / C::BK;
    const int wb = (int)((int64_t)slice * nwin / slices);
    const int we = (int)((int64_t)(slice + 1) * nwin / slices);
    Acc<C> acc;
    zero_acc<C>(acc);
    mma_tile<C>(g, lds, m0, n0, wb, we, acc);
    const int r_first = KwReduce<C>::run(lds, acc);
    GemmArgs o = g;
    o.C = ws + (int64_t)slice * g.M * g.N;
    o.ldc = g.N;
    o.alpha = 1.0f;
    o.beta = 0.0f;
    store_tile<C>(o, m0, n0, acc, m_lo, n_lo, r_first, KwReduce<C>::RPG);
}

// Whether a launch of `blocks` work-groups, each over `windows` k windows, uses
// the tile's register ring.  The ring lets a block's loads run several windows
// ahead, which pays when the wait for each window's loads sets the pace: one
// round of blocks over a long k (1024^3 on 64 x 64 blocks -9%, 512 x 512 x 32768
// on 32 x 32 x 64 blocks -25%), or several rounds over a very long one (256 x
// 8192 x 8192, 256 windows in two rounds, -7%; 1000 x 5000 x 2000, 125 windows
// in five rounds, -5%).  It costs a longer prologue and more guarded windows at
// the end, which lose on short k (4096 x 4096 x 256 on 128 x 128 blocks, 16
// windows, +14%) and on grids of several rounds over a moderate k (6000 x 6000
// x 1000, 63 windows, +3%; 4095 x 4097 x 1023 on 192 x 128 blocks +1.4%).
template <class T>
bool use_ring(int64_t blocks, int64_t windows) {
    return T::RING > 1 && windows >= 16 && (blocks <= compute_units() || windows >= 96);
}

template <class T, bool TA, bool TB, int R>
hipError_t launch_tile_r(const Problem &p, hipStream_t s, int64_t tiles_m, int64_t tiles_n) {
    const GemmArgs g{p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.alpha, p.beta};
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(T::THREADS);
    if (narrow_offsets<T, TA, TB>(p))
        return launch(mfma_kernel<Cfg<T, TA, TB, true, R>>, grid, block, 0, s, g, (int)tiles_m,
                      (int)tiles_n);
    return launch(mfma_kernel<Cfg<T, TA, TB, false, R>>, grid, block, 0, s, g, (int)tiles_m,
                  (int)tiles_n);
}

template <class T, bool TA, bool TB>
hipError_t launch_tile(const Problem &p, hipStream_t s) {
    const int64_t tiles_m = (p.M + T::BM - 1) / T::BM;
    const int64_t tiles_n = (p.N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n > INT32_MAX) return hipErrorInvalidValue;
    if constexpr (T::RING > 1) {
        if (use_ring<T>(tiles_m * tiles_n, ((int64_t)p.K + T::BK - 1) / T::BK))
            return launch_tile_r<T, TA, TB, T::RING>(p, s, tiles_m, tiles_n);
    }
    return launch_tile_r<T, TA, TB, 1>(p, s, tiles_m, tiles_n);
}

// The split-k form of configuration T with `slices` slices; the caller has checked
// that every slice holds at least one k window and that the workspace holds
// slices * M * N floats.
template <class T, bool TA, bool TB, int R>
hipError_t launch_tile_splitk_r(const Problem &p, hipStream_t s, int slices, float *ws,
                                int64_t tiles_m, int64_t tiles_n) {
    const GemmArgs g{p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.alpha, p.beta};
    const dim3 grid((unsigned)(tiles_m * tiles_n * slices)), block(T::THREADS);
    if (narrow_offsets<T, TA, TB>(p))
        return launch(mfma_splitk_kernel<Cfg<T, TA, TB, true, R>>, grid, block, 0, s, g,
                      (int)tiles_m, (int)tiles_n, slices, ws);
    return launch(mfma_splitk_kernel<Cfg<T, TA, TB, false, R>>, grid, block, 0, s, g,
                  (int)tiles_m, (int)tiles_n, slices, ws);
}

template <class T, bool TA, bool TB>
hipError_t launch_tile_splitk(const Problem &p, hipStream_t s, int slices, float *ws) {
    const int64_t tiles_m = (p.M + T::BM - 1) / T::BM;
    const int64_t tiles_n = (p.N + T::BN - 1) / T::BN;
    if (tiles_m * tiles_n * slices > INT32_MAX) return hipErrorInvalidValue;
    if constexpr (T::RING > 1) {
        const int64_t windows = ((int64_t)p.K + T::BK - 1) / T::BK / slices;
        if (use_ring<T>(tiles_m * tiles_n * slices, windows))
            return launch_tile_splitk_r<T, TA, TB, T::RING>(p, s, slices, ws, tiles_m, tiles_n);
    }
    return launch_tile_splitk_r<T, TA, TB, 1>(p, s, slices, ws, tiles_m, tiles_n);
}

// ---------------------------------------------------------------------------
// Tile configurations.
// 256 x 256 blocks, one wave per SIMD with 128 x 128 of C each: large products.
using TileHuge = MfmaTile<256, 256, 16, 128, 128, 1, 8, 3>;
using TileWide = MfmaTile<128, 128, 16, 32, 128, 1, 8, 3, 1, 4, 8, 3>;
// 128 x 192 blocks of 64 x 96 per wave, k split over two wave groups (two waves
// per SIMD): one block per CU on grids of about 256 blocks, such as 2048 x 3072.
using TileSplit192 = MfmaTile<128, 192, 32, 64, 96, 2, 8, 3>;
// The same block as eight waves of 32 x 96 without the k split (two waves per
// SIMD), in its place when only B is transposed: B's fragments are then one
// 16-byte read per 32-wide block, and 2048 x 3072 x 4096 ran at 146.2 against
// 144.5 TFLOP/s, other shapes on this block 1.0-3.1% faster.  With B as given
// the two measured within 0.3% at 2048 x 3072 x 4096 and 2000 x 3001 x 4000
// (1.6% faster at 1999 x 2999 x 1000; TileSplit192 kept); with A transposed a
// 32-high wave reads A one float per k and was 1.7% (B transposed too) and 4.2%
// slower.
using TileWide192 = MfmaTile<128, 192, 32, 32, 96, 1, 8, 3>;
template <bool TA, bool TB>
using Tile192 = typename std::conditional<!TA && TB, TileWide192, TileSplit192>::type;
// 192 x 128 blocks of 96 x 64 per wave.
using TileTall = MfmaTile<192, 128, 16, 96, 64, 1, 8, 3, 1, 4, 8, 3>;
using TileSmall = MfmaTile<64, 64, 16, 32, 32, 1, 4, 3, 1, 4, 8, 3>;
using TileSplit64 = MfmaTile<64, 64, 32, 32, 32, 2, 4, 3, 1, 4, 8, 3>;
// k split four ways: one 8-wide step per group and window, so two stages.
using TileTiny = MfmaTile<32, 32, 32, 32, 32, 4, 4, 2, 1, 4, 8, 2>;
// The same block with 64-wide windows and three stages: twice the work per
// window and one more window in flight, for grids of at most one block per CU
// over a long k, where TileTiny waits on its loads (512 x 512 x 32768: 352 ->
// 230 us).  Its 57 KB of LDS allow two blocks per CU, so many-block grids stay
// with TileTiny.
using TileTiny64 = MfmaTile<32, 32, 64, 32, 32, 4, 4, 3, 1, 4, 8, 3>;

constexpr int kTileCount = 8;

// Launch configuration `tile` (0 <= tile < kTileCount, in the order above) for
// one storage order (defined in mfma_nn.hip, mfma_nt.hip, mfma_tn.hip, mfma_tt.hip).
hipError_t launch_mfma_nn(const Problem &p, hipStream_t s, int tile);
hipError_t launch_mfma_nt(const Problem &p, hipStream_t s, int tile);
hipError_t launch_mfma_tn(const Problem &p, hipStream_t s, int tile);
hipError_t launch_mfma_tt(const Problem &p, hipStream_t s, int tile);
// Split-k launches of the configurations that split-k uses (TileWide, TileSmall,
// TileSplit64); hipErrorInvalidValue for the others.
hipError_t launch_mfma_nn_splitk(const Problem &p, hipStream_t s, int tile, int slices, float *ws);
hipError_t launch_mfma_nt_splitk(const Problem &p, hipStream_t s, int tile, int slices, float *ws);
hipError_t launch_mfma_tn_splitk(const Problem &p, hipStream_t s, int tile, int slices, float *ws);
hipError_t launch_mfma_tt_splitk(const Problem &p, hipStream_t s, int tile, int slices, float *ws);

#define SGEMM_MFMA_LAUNCHER(NAME, TA, TB)                                                     \
    hipError_t NAME(const Problem &p, hipStream_t s, int tile) {                             \
        switch (tile) {                                                                       \
        case 0: return launch_tile<TileHuge, TA, TB>(p, s);                                   \
        case 1: return launch_tile<TileWide, TA, TB>(p, s);                                   \
        case 2: return launch_tile<Tile192<TA, TB>, TA, TB>(p, s);                            \
        case 3: return launch_tile<TileTall, TA, TB>(p, s);                                   \
        case 4: return launch_tile<TileSmall, TA, TB>(p, s);                                  \
        case 5: return launch_tile<TileSplit64, TA, TB>(p, s);                                \
        case 6: return launch_tile<TileTiny, TA, TB>(p, s);                                   \
        case 7: return launch_tile<TileTiny64, TA, TB>(p, s);                                 \
        default: return hipErrorInvalidValue;                                                 \
        }                                                                                     \
    }                                                                                         \
    hipError_t NAME##_splitk(const Problem &p, hipStream_t s, int tile, int slices, float *ws) { \
        switch (tile) {                                                                       \
        case 1: return launch_tile_splitk<TileWide, TA, TB>(p, s, slices, ws);                \
        case 4: return launch_tile_splitk<TileSmall, TA, TB>(p, s, slices, ws);               \
        case 5: return launch_tile_splitk<TileSplit64, TA, TB>(p, s, slices, ws);             \
        default: return hipErrorInvalidValue;                                                 \
        }                                                                                     \
    }

}  // namespace sgemm
