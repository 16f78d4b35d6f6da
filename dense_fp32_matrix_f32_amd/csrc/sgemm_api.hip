// sgemm_api.hip -- the C ABI of include/sgemm_f32.h: argument validation on the
// host (before any HIP call), choice of kernel, and launch on the caller's stream.
#include "sgemm_f32.h"

#include <atomic>
#include <mutex>

#include "internal.h"

using sgemm::Problem;

namespace {

// Byte extent [lo, hi) of a rows x cols row-major array with row stride ld
// (rows, cols, ld >= 1).  Sizes near the int range make the byte count exceed
// 64 bits, so it is formed in 128 bits and hi saturates at the top of the
// address space rather than wrapping below lo.
struct Extent {
    uintptr_t lo, hi;
};

Extent extent(const void *p, int64_t rows, int64_t cols, int64_t ld) {
    const uintptr_t lo = (uintptr_t)p;
    const unsigned __int128 bytes =
        ((unsigned __int128)(uint64_t)(rows - 1) * (uint64_t)ld + (uint64_t)cols) * sizeof(float);
    const unsigned __int128 hi = (unsigned __int128)lo + bytes;
    return {lo, hi > (unsigned __int128)UINTPTR_MAX ? UINTPTR_MAX : (uintptr_t)hi};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

int at_least_one(int x) { return x > 1 ? x : 1; }

// hipSuccess if the arguments describe a valid C = alpha*op(A)*op(B) + beta*C,
// else hipErrorInvalidValue.  A and B are read only when alpha != 0 and K > 0.
hipError_t validate(int transa, int transb, int M, int N, int K, float alpha, const float *A,
                    int lda, const float *B, int ldb, const float *C, int ldc) {
    if ((transa != SGEMM_F32_OP_N && transa != SGEMM_F32_OP_T) ||
        (transb != SGEMM_F32_OP_N && transb != SGEMM_F32_OP_T))
        return hipErrorInvalidValue;
    if (M < 0 || N < 0 || K < 0) return hipErrorInvalidValue;
    if (lda < at_least_one(transa ? M : K) || ldb < at_least_one(transb ? K : N) ||
        ldc < at_least_one(N))
        return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    if (C == nullptr) return hipErrorInvalidValue;
    if (K == 0 || alpha == 0.0f) return hipSuccess;
    if (A == nullptr || B == nullptr) return hipErrorInvalidValue;
    const Extent c = extent(C, M, N, ldc);
    const Extent a = transa ? extent(A, K, M, lda) : extent(A, M, K, lda);
    const Extent b = transb ? extent(B, N, K, ldb) : extent(B, K, N, ldb);
    if (overlaps(c, a) || overlaps(c, b)) return hipErrorInvalidValue;
    return hipSuccess;
}

// Products with few rows or few columns stream one operand and are bound by
// memory, so the streaming kernels win; everything else goes to the matrix
// cores.
int choose(int transa, int transb, int M, int N, int K) {
    (void)K;
    if (M <= 8) return SGEMM_F32_ALGO_SKINNY;
    if (N <= 8) return SGEMM_F32_ALGO_SKINNY_N;
    // With A transposed and B not, both operands run along m or n, so a product
    // narrower than one 32-wide block of the matrix cores in m or n loads that
    // operand element by element there; two or three passes of the streaming
    // kernels are faster up to 24 (12 x 4096 x 4096: 33.9 against 60.4 us,
    // 24 x 4096 x 4096: 54.4 against 60.4, 4096 x 16 x 4096: 37.3 against 66.0).
    if (transa == SGEMM_F32_OP_T && transb == SGEMM_F32_OP_N) {
        if (M <= 24) return SGEMM_F32_ALGO_SKINNY;
        if (N <= 24) return SGEMM_F32_ALGO_SKINNY_N;
    }
    return SGEMM_F32_ALGO_MFMA;
}

// Few rows (columns) of C in any storage order: the streaming kernel whose
// streamed operand runs along memory (see internal.h).
hipError_t launch_few_rows(const Problem &p, hipStream_t s) {
    return p.tb ? sgemm::launch_skinny_rows_tb(p, s) : sgemm::launch_skinny_rows(p, s);
}

hipError_t launch_few_cols(const Problem &p, hipStream_t s) {
    return p.ta ? sgemm::launch_skinny_cols_ta(p, s) : sgemm::launch_skinny_cols(p, s);
}

// Automatic choice for the products the matrix cores take.  When N lies a few
// columns past a multiple of 32 (M a few rows), those columns (rows) need a whole
// extra column (row) of blocks of C, which can add a round of blocks on the CUs
// for a sliver of work (4095 x 4097: 726 blocks of 192 x 128 for 4095 x 4096
// plus one column).  The product is then split: the blocks cover the leading
// multiple of 32 and the strip that is left goes to a kernel sized for it (the
// streaming kernels), when the cost model of the tile table says the launches
// together finish sooner.
// Every element of C is still computed whole by exactly one kernel.
constexpr int kPeelMax = 8;    // widest strip split off
constexpr double kStreamBytesPerUs = 2.5e6;  // streaming kernels on small strips
constexpr double kStreamLaunchUs = 4.0;

// Modelled time of a rows x cols strip over the whole k range.
double strip_us(const Problem &p, int rows, int cols) {
    const double bytes = 4.0 * ((double)rows * p.K + (double)p.K * cols + (double)rows * cols);
    return kStreamLaunchUs + bytes / kStreamBytesPerUs;
}

hipError_t launch_strip(const Problem &q, hipStream_t s) {
    return q.M <= kPeelMax ? launch_few_rows(q, s) : launch_few_cols(q, s);
}

// Columns [n0, N) of op(B) and C, all rows.
Problem column_strip(const Problem &p, int n0) {
    Problem q = p;
    q.N = p.N - n0;
    q.B = p.tb ? p.B + (int64_t)n0 * p.ldb : p.B + n0;
    q.C = p.C + n0;
    return q;
}

// Rows [m0, M) of op(A) and C, columns [0, n_end).
Problem row_strip(const Problem &p, int m0, int n_end) {
    Problem q = p;
    q.M = p.M - m0;
    q.N = n_end;
    q.A = p.ta ? p.A + m0 : p.A + (int64_t)m0 * p.lda;
    q.C = p.C + (int64_t)m0 * p.ldc;
    return q;
}

// Extents of the part of C that the blocks cover; the rest (columns
// [n_main, N), then rows [m_main, M) of columns [0, n_main)) goes to strips.
struct Split {
    int m_main, n_main;
};

Split plan_split(const Problem &p, int cus) {
    Split full{p.M, p.N};
    const int rn = p.N % 32, rm = p.M % 32;
    const bool cut_n = p.N >= 64 && rn >= 1 && rn <= kPeelMax;
    const bool cut_m = p.M >= 64 && rm >= 1 && rm <= kPeelMax;
    if (!cut_n && !cut_m) return full;
    const double full_us = sgemm::mfma_model_us(p.M, p.N, p.K, cus);
    Split best = full;
    double best_us = full_us;
    // bit 0 splits off the last rn columns, bit 1 the last rm rows
    for (int plan = 1; plan < 4; ++plan) {
        const bool pn = plan & 1, pm = plan & 2;
        if ((pn && !cut_n) || (pm && !cut_m)) continue;
        const Split sp{pm ? p.M - rm : p.M, pn ? p.N - rn : p.N};
        double us = sgemm::mfma_model_us(sp.m_main, sp.n_main, p.K, cus);
        if (pn) us += strip_us(p, p.M, rn);
        if (pm) us += strip_us(p, rm, sp.n_main);
        if (us < best_us) {
            best = sp;
            best_us = us;
        }
    }
    return best_us <= 0.97 * full_us ? best : full;
}

hipError_t launch_auto_mfma(const Problem &p, hipStream_t s) {
    const Split sp = plan_split(p, sgemm::compute_units());
    Problem main = p;
    main.M = sp.m_main;
    main.N = sp.n_main;
    hipError_t e = sgemm::launch_mfma(main, s);
    if (e == hipSuccess && sp.n_main < p.N) e = launch_strip(column_strip(p, sp.n_main), s);
    if (e == hipSuccess && sp.m_main < p.M) e = launch_strip(row_strip(p, sp.m_main, sp.n_main), s);
    return e;
}

// ---------------------------------------------------------------------------
// Split-k with a caller-provided workspace.  Products with few blocks of C and a
// long k leave most CUs idle (128 x 128 x 65536: 4 blocks of 64 x 64); they split
// k into slices whose unscaled partial products go to workspace planes, added by
// a second kernel in an order fixed by the shape (deterministic, no atomics).
// The few-rows kernel was tried the same way (row segments of 512 bytes to 4 KiB
// for 1 x 4096 x 4096): the partial sums alone read B as fast as a contiguous
// copy, but adding them, by a second launch or by the last group to arrive,
// costs more than the strips lose, so it never splits.
enum WsKind { WS_NONE = 0, WS_MFMA = 1 };
struct WsPlan {
    int kind, tile, slices;
};

// Cost of the partial planes beyond the product kernel: the planes are written
// by the product kernel and read back by the reduction (fitted on the same split
// launches as the product model: 2.5 us fixed, 0.31 us per MB of planes), and at
// most 64 MiB of planes, which stay in the Infinity Cache between the two.
constexpr double kSplitFixedUs = 2.5;
constexpr double kSplitUsPerMB = 0.31;
constexpr int64_t kSplitMaxPlaneBytes = 64ll << 20;

double split_overhead_us(const Problem &p, int slices) {
    const double plane = 4.0 * p.M * (double)p.N;
    return kSplitFixedUs + (slices * plane + plane * (p.beta != 0.0f ? 2 : 1)) * kSplitUsPerMB / 1e6;
}

int64_t ws_bytes(const WsPlan &w, const Problem &p) {
    return w.kind == WS_NONE ? 0 : (int64_t)w.slices * p.M * p.N * (int64_t)sizeof(float);
}

WsPlan plan_workspace(const Problem &p, int algo, int cus) {
    WsPlan none{WS_NONE, 0, 1};
    if (p.M == 0 || p.N == 0 || p.K == 0 || algo != SGEMM_F32_ALGO_MFMA) return none;
    const double whole = sgemm::mfma_model_us(p.M, p.N, p.K, cus);
    WsPlan best = none;
    double best_us = whole;
    static constexpr int kSplitTiles[] = {1, 4, 5};
    for (int tile : kSplitTiles) {
        const int64_t nwin = ((int64_t)p.K + sgemm::mfma_tile_bk(tile) - 1) / sgemm::mfma_tile_bk(tile);
        for (int slices = 2; slices <= 128 && 2 * (int64_t)slices <= nwin &&
                             (int64_t)slices * p.M * p.N * 4 <= kSplitMaxPlaneBytes;
             slices *= 2) {
            const double us = sgemm::mfma_model_tile_us(tile, p.M, p.N, p.K, cus, slices) +
                              split_overhead_us(p, slices);
            if (us < best_us) {
                best_us = us;
                best = WsPlan{WS_MFMA, tile, slices};
            }
        }
    }
    return best_us < 0.9 * whole ? best : none;
}

// The two kernels of a split product: partial planes to `planes`, then the
// fixed-order reduction into C.
hipError_t launch_split_planes(const Problem &p, const WsPlan &w, float *planes,
                               hipStream_t stream) {
    const hipError_t st = sgemm::launch_mfma_splitk(p, stream, w.tile, w.slices, planes);
    if (st != hipSuccess) return st;
    return sgemm::launch_splitk_reduce(p, w.slices, planes, stream);
}

// ---------------------------------------------------------------------------
// Split-k for callers that cannot allocate: the planes go to a file-scope device
// array of SGEMM_F32_SCRATCH_BYTES.  Each GPU the library runs on holds its own
// copy, at its own address, until the process ends.  On the host the array's
// name is not a device address, so its address on each device is looked up once
// (with that device current) and kept; kernels only ever see that address.
static __device__ __align__(256) float scratch[SGEMM_F32_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_addr[kMaxDevices];
std::mutex scratch_lookup;

// Address of the current device's copy of `scratch`.
hipError_t scratch_on_current_device(float **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *ptr = scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> hold(scratch_lookup);
        ptr = scratch_addr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (ptr == nullptr) return hipErrorInvalidSymbol;
            scratch_addr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = (float *)ptr;
    return hipSuccess;
}

bool handles_transposes(int algo) {
    return algo == SGEMM_F32_ALGO_AUTO || algo == SGEMM_F32_ALGO_NAIVE ||
           algo == SGEMM_F32_ALGO_LDS_TILED || algo == SGEMM_F32_ALGO_MFMA ||
           algo == SGEMM_F32_ALGO_SKINNY || algo == SGEMM_F32_ALGO_SKINNY_N;
}

Problem problem(int transa, int transb, int M, int N, int K, float alpha, const float *A,
                int lda, const float *B, int ldb, float beta, float *C, int ldc) {
    Problem p{M, N, K, A, lda, B, ldb, C, ldc};
    p.ta = transa == SGEMM_F32_OP_T;
    p.tb = transb == SGEMM_F32_OP_T;
    p.alpha = alpha;
    p.beta = beta;
    return p;
}

// Validation and the product-free cases shared by the entry points.  Returns
// true with *status set when nothing is left to launch.
bool trivial(int transa, int transb, int M, int N, int K, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream,
             hipError_t *status) {
    *status = validate(transa, transb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (*status != hipSuccess) return true;
    if (M == 0 || N == 0) return true;
    if (K == 0 || alpha == 0.0f) {
        *status = sgemm::launch_scale(
            problem(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc), stream);
        return true;
    }
    return false;
}

}  // namespace

extern "C" const char *sgemm_f32_algo_name(int algo) {
    switch (algo) {
    case SGEMM_F32_ALGO_AUTO: return "auto";
    case SGEMM_F32_ALGO_NAIVE: return "naive";
    case SGEMM_F32_ALGO_LDS_TILED: return "lds_tiled";
    case SGEMM_F32_ALGO_VALU_REGBLOCK: return "valu_regblock";
    case SGEMM_F32_ALGO_MFMA: return "mfma";
    case SGEMM_F32_ALGO_SKINNY: return "skinny";
    case SGEMM_F32_ALGO_SKINNY_N: return "skinny_n";
    case SGEMM_F32_ALGO_BF16X6: return "bf16x6";
    default: return "invalid";
    }
}

extern "C" int sgemm_f32_select(int M, int N, int K, const float *A, int lda, const float *B,
                                int ldb, const float *C, int ldc) {
    if (validate(SGEMM_F32_OP_N, SGEMM_F32_OP_N, M, N, K, 1.0f, A, lda, B, ldb, C, ldc) !=
        hipSuccess)
        return -1;
    return choose(SGEMM_F32_OP_N, SGEMM_F32_OP_N, M, N, K);
}

extern "C" int sgemm_f32_auto_plan(int transa, int transb, int M, int N, int K,
                                   int compute_units, int *m_main, int *n_main) {
    if ((transa != SGEMM_F32_OP_N && transa != SGEMM_F32_OP_T) ||
        (transb != SGEMM_F32_OP_N && transb != SGEMM_F32_OP_T) || M < 0 || N < 0 || K < 0 ||
        m_main == nullptr || n_main == nullptr)
        return -1;
    const int algo = choose(transa, transb, M, N, K);
    Split sp{M, N};
    if (algo == SGEMM_F32_ALGO_MFMA && M > 0 && N > 0 && K > 0) {
        Problem p{M, N, K, nullptr, 1, nullptr, 1, nullptr, 1};
        p.ta = transa == SGEMM_F32_OP_T;
        p.tb = transb == SGEMM_F32_OP_T;
        sp = plan_split(p, compute_units > 0 ? compute_units : 256);
    }
    *m_main = sp.m_main;
    *n_main = sp.n_main;
    return algo;
}

extern "C" hipError_t sgemm_f32_ex_algo(int transa, int transb, int M, int N, int K, float alpha,
                                        const float *A, int lda, const float *B, int ldb,
                                        float beta, float *C, int ldc, hipStream_t stream,
                                        int algo) {
    if (algo < 0 || algo >= SGEMM_F32_ALGO_COUNT) return hipErrorInvalidValue;
    if ((transa == SGEMM_F32_OP_T || transb == SGEMM_F32_OP_T) && !handles_transposes(algo))
        return hipErrorInvalidValue;
    hipError_t st;
    if (trivial(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, &st))
        return st;
    const Problem p = problem(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    if (algo == SGEMM_F32_ALGO_AUTO) {
        algo = choose(transa, transb, M, N, K);
        if (algo == SGEMM_F32_ALGO_MFMA) return launch_auto_mfma(p, stream);
    }
    switch (algo) {
    case SGEMM_F32_ALGO_NAIVE: return sgemm::launch_naive(p, stream);
    case SGEMM_F32_ALGO_LDS_TILED: return sgemm::launch_lds_tiled(p, stream);
    case SGEMM_F32_ALGO_VALU_REGBLOCK: return sgemm::launch_valu_regblock(p, stream);
    case SGEMM_F32_ALGO_MFMA: return sgemm::launch_mfma(p, stream);
    case SGEMM_F32_ALGO_SKINNY: return launch_few_rows(p, stream);
    case SGEMM_F32_ALGO_SKINNY_N: return launch_few_cols(p, stream);
    case SGEMM_F32_ALGO_BF16X6: return sgemm::launch_split(p, stream);
    default: return hipErrorInvalidValue;
    }
}

extern "C" size_t sgemm_f32_workspace_size(int transa, int transb, int M, int N, int K) {
    if ((transa != SGEMM_F32_OP_N && transa != SGEMM_F32_OP_T) ||
        (transb != SGEMM_F32_OP_N && transb != SGEMM_F32_OP_T) || M < 0 || N < 0 || K < 0)
        return 0;
    Problem p{M, N, K, nullptr, 1, nullptr, 1, nullptr, 1};
    p.ta = transa == SGEMM_F32_OP_T;
    p.tb = transb == SGEMM_F32_OP_T;
    const WsPlan w = plan_workspace(p, choose(transa, transb, M, N, K), sgemm::compute_units());
    return (size_t)ws_bytes(w, p);
}

extern "C" hipError_t sgemm_f32_ex_ws(int transa, int transb, int M, int N, int K, float alpha,
                                      const float *A, int lda, const float *B, int ldb,
                                      float beta, float *C, int ldc, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    hipError_t st;
    if (trivial(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, &st))
        return st;
    if (workspace != nullptr && workspace_bytes > 0 && ((uintptr_t)workspace & 15) != 0)
        return hipErrorInvalidValue;
    const Problem p = problem(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    const int algo = choose(transa, transb, M, N, K);
    const WsPlan w = plan_workspace(p, algo, sgemm::compute_units());
    const int64_t need = ws_bytes(w, p);
    if (w.kind == WS_NONE || workspace == nullptr || (uint64_t)need > workspace_bytes)
        return sgemm_f32_ex(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
    // the part of the workspace used must not overlap the operands or C
    const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + (uintptr_t)need};
    const Extent c = extent(C, M, N, ldc);
    const Extent a = transa ? extent(A, K, M, lda) : extent(A, M, K, lda);
    const Extent b = transb ? extent(B, N, K, ldb) : extent(B, K, N, ldb);
    if (overlaps(ws, a) || overlaps(ws, b) || overlaps(ws, c)) return hipErrorInvalidValue;
    return launch_split_planes(p, w, (float *)workspace, stream);
}

extern "C" hipError_t sgemm_f32_ex_noalloc(int transa, int transb, int M, int N, int K,
                                           float alpha, const float *A, int lda, const float *B,
                                           int ldb, float beta, float *C, int ldc,
                                           hipStream_t stream) {
    hipError_t st;
    if (trivial(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, &st))
        return st;
    const Problem p = problem(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    const WsPlan w = plan_workspace(p, choose(transa, transb, M, N, K), sgemm::compute_units());
    if (w.kind == WS_NONE)
        return sgemm_f32_ex(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
    if ((uint64_t)ws_bytes(w, p) > SGEMM_F32_SCRATCH_BYTES) return hipErrorInvalidValue;
    float *planes = nullptr;
    st = scratch_on_current_device(&planes);
    if (st != hipSuccess) return st;
    // the scratch array is the library's own, so it cannot overlap A, B or C
    return launch_split_planes(p, w, planes, stream);
}

extern "C" hipError_t sgemm_f32_ex(int transa, int transb, int M, int N, int K, float alpha,
                                   const float *A, int lda, const float *B, int ldb, float beta,
                                   float *C, int ldc, hipStream_t stream) {
    return sgemm_f32_ex_algo(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                             SGEMM_F32_ALGO_AUTO);
}

extern "C" hipError_t sgemm_f32_algo(int M, int N, int K, const float *A, int lda,
                                     const float *B, int ldb, float *C, int ldc,
                                     hipStream_t stream, int algo) {
    return sgemm_f32_ex_algo(SGEMM_F32_OP_N, SGEMM_F32_OP_N, M, N, K, 1.0f, A, lda, B, ldb, 0.0f,
                             C, ldc, stream, algo);
}

extern "C" hipError_t sgemm_f32(int M, int N, int K, const float *A, int lda, const float *B,
                                int ldb, float *C, int ldc, hipStream_t stream) {
    return sgemm_f32_algo(M, N, K, A, lda, B, ldb, C, ldc, stream, SGEMM_F32_ALGO_AUTO);
}

extern "C" hipError_t sgemm_f32_colmajor(int transa, int transb, int M, int N, int K,
                                         float alpha, const float *A, int lda, const float *B,
                                         int ldb, float beta, float *C, int ldc,
                                         hipStream_t stream) {
    // A column-major array is the row-major array of its transpose, so
    // C^T = alpha*op(B)^T*op(A)^T + beta*C^T in row-major terms.
    return sgemm_f32_ex(transb, transa, N, M, K, alpha, B, ldb, A, lda, beta, C, ldc, stream);
}

extern "C" int sgemm_f32_mfma_tiles(void) { return sgemm::mfma_tile_count(); }

extern "C" const char *sgemm_f32_mfma_tile_name(int tile) { return sgemm::mfma_tile_name(tile); }

extern "C" int sgemm_f32_mfma_select(int M, int N, int K, int compute_units) {
    if (M < 0 || N < 0 || K < 0) return -1;
    return sgemm::mfma_select(M, N, K, compute_units);
}

extern "C" hipError_t sgemm_f32_ex_mfma_tile(int transa, int transb, int M, int N, int K,
                                             float alpha, const float *A, int lda,
                                             const float *B, int ldb, float beta, float *C,
                                             int ldc, hipStream_t stream, int tile) {
    if (tile < 0 || tile >= sgemm::mfma_tile_count()) return hipErrorInvalidValue;
    hipError_t st;
    if (trivial(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, &st))
        return st;
    return sgemm::launch_mfma_tile(
        problem(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc), stream, tile);
}

extern "C" hipError_t sgemm_f32_mfma_tile(int M, int N, int K, const float *A, int lda,
                                          const float *B, int ldb, float *C, int ldc,
                                          hipStream_t stream, int tile) {
    return sgemm_f32_ex_mfma_tile(SGEMM_F32_OP_N, SGEMM_F32_OP_N, M, N, K, 1.0f, A, lda, B, ldb,
                                  0.0f, C, ldc, stream, tile);
}
