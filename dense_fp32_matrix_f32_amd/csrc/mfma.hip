// mfma.hip -- the matrix-core rung: tile table, cost-model choice and dispatch
// to the kernels of mfma_kernel.h (instantiated per operand storage order in
// mfma_nn.hip, mfma_nt.hip, mfma_tn.hip and mfma_tt.hip).
#include <atomic>
#include <cmath>

#include "mfma_kernel.h"

namespace sgemm {

// ---------------------------------------------------------------------------
// Tile choice.  A launch of T tiles on U compute units finishes when the busiest
// CU has worked through R = ceil(T / U) tiles, so a configuration's time is
// modelled as R * (2*BM*BN*K / (e / 256) + t1) + t0, where e is a whole-chip
// throughput in TFLOP/s, t1 a fixed cost per tile (prologue, epilogue) and t0 a
// fixed cost per launch.  Each configuration has two throughputs: one for
// products whose A and B together fit in 200 MB (inside the 256 MB Infinity
// Cache), one for larger products.  When every CU gets at most one block, the
// per-block term is at least the block's k windows times a per-window latency
// (window_floor_us below).  The four numbers per configuration were fitted
// (least squares on log time) to timings of every configuration on 19 shapes on
// MI355X, among them the 512^3, 1024^3, 2048 x 3072 x 4096, 4095 x 4097 x 1023
// and 8192^3 products and four with a long k and few blocks.  The fit predates
// the register ring of the kernels and their stage-unrolled loops; timed again
// on the current kernels, the model picks the fastest configuration on 15 of the
// 19 shapes and one within 2.4% of it on the other four (4095 x 4097 x 1023 over
// the whole shape, 4096 x 4096 x 256, 256 x 8192 x 8192, 8192 x 256 x 8192), so
// the numbers were kept.  The smallest estimate wins.  The timings are of
// untransposed operands; the other storage orders use the same choice.
struct TileChoice {
    const char *name;  // block, k window, wave block, wave groups, LDS stages
    int bm, bn;
    double tflops_cached;  // e, A and B within 200 MB
    double tflops_large;   // e, larger A and B
    double t0_us;          // t0
    double t1_us;          // t1
};

static constexpr TileChoice kTiles[] = {
    {"256x256x16 w128x128 k1 s3", 256, 256, 150.5, 151.0, 0.0, 16.0},
    {"128x128x16 w32x128 k1 s3", 128, 128, 146.5, 145.5, 5.5, 2.0},
    {"128x192x32 w64x96 k2 s3", 128, 192, 144.5, 146.0, 6.0, 8.0},
    {"192x128x16 w96x64 k1 s3", 192, 128, 147.0, 146.5, 8.5, 3.0},
    {"64x64x16 w32x32 k1 s3", 64, 64, 125.5, 121.0, 8.5, 0.0},
    {"64x64x32 w32x32 k2 s3", 64, 64, 126.5, 126.0, 6.0, 1.0},
    {"32x32x32 w32x32 k4 s2", 32, 32, 105.5, 106.0, 6.5, 0.0},
    {"32x32x64 w32x32 k4 s3", 32, 32, 116.0, 106.5, 6.0, 2.0},
};
static_assert(sizeof(kTiles) / sizeof(kTiles[0]) == kTileCount, "one entry per configuration");
// The table rows follow the launcher tables of mfma_kernel.h.
static_assert(kTiles[0].bm == TileHuge::BM && kTiles[0].bn == TileHuge::BN, "row 0");
static_assert(kTiles[1].bm == TileWide::BM && kTiles[1].bn == TileWide::BN, "row 1");
static_assert(kTiles[2].bm == TileSplit192::BM && kTiles[2].bn == TileSplit192::BN, "row 2");
static_assert(TileWide192::BM == TileSplit192::BM && TileWide192::BN == TileSplit192::BN &&
                  TileWide192::BK == TileSplit192::BK,
              "row 2 in both wave shapes");
static_assert(kTiles[3].bm == TileTall::BM && kTiles[3].bn == TileTall::BN, "row 3");
static_assert(kTiles[4].bm == TileSmall::BM && kTiles[4].bn == TileSmall::BN, "row 4");
static_assert(kTiles[5].bm == TileSplit64::BM && kTiles[5].bn == TileSplit64::BN, "row 5");
static_assert(kTiles[6].bm == TileTiny::BM && kTiles[6].bn == TileTiny::BN, "row 6");
static_assert(kTiles[7].bm == TileTiny64::BM && kTiles[7].bn == TileTiny64::BN, "row 7");

// Compute units of the current device, looked up once per device (256 if the
// query fails, as on a host without a GPU).
int compute_units() {
    static std::atomic<int> known[64];
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64 && (cus = known[dev].load(std::memory_order_relaxed)) > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    if (dev >= 0 && dev < 64) known[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// A work-group cannot go faster than its chain of k windows allows: each window
// waits for loads that were issued a fixed number of windows earlier.  With one
// work-group per CU nothing else hides that wait, and configurations with little
// arithmetic per window (32 x 32 blocks) run at about half their throughput on
// long k.  Measured per window: about 0.18 us while A and B fit in 8 MiB (the
// L2 caches), 0.34 us for larger operands.
static double window_floor_us(double operand_bytes) {
    return operand_bytes <= 8.0 * 1024 * 1024 ? 0.18 : 0.34;
}

static double per_cu_rate(const TileChoice &c, double operand_bytes) {
    return (operand_bytes <= 200e6 ? c.tflops_cached : c.tflops_large) / 256.0;  // fitted on 256 CUs
}

// Modelled time of configuration i on the whole k range.
static double tile_us(int i, int M, int N, int K, int cus) {
    const TileChoice &c = kTiles[i];
    const double tiles = (double)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const double per_cu = std::ceil(tiles / cus);
    const double operands = 4.0 * ((double)M * K + (double)K * N);
    double work = 2.0 * c.bm * c.bn * (double)K / (per_cu_rate(c, operands) * 1e6);
    if (per_cu == 1) {
        const double windows = std::ceil((double)K / mfma_tile_bk(i));
        work = std::fmax(work, windows * window_floor_us(operands));
    }
    return per_cu * (work + c.t1_us) + c.t0_us;
}

// Modelled time of the product kernel of configuration i with the k windows
// split into `slices` slices (tiles * slices work-groups over K / slices each).
// Fitted separately on split launches (20 shapes, 3 configurations, 2..128
// slices): work-groups of short k overlap their prologue and epilogue with the
// other work-group resident on the CU, so t1 is paid once, not per round, and
// the window floor applies to every second round.
static double split_tile_us(int i, int M, int N, int K, int cus, int slices) {
    const TileChoice &c = kTiles[i];
    const double tiles = (double)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * slices;
    const double per_cu = std::ceil(tiles / cus);
    const double operands = 4.0 * ((double)M * K + (double)K * N);
    const double k_slice = std::ceil((double)K / slices);
    const double work = per_cu * 2.0 * c.bm * c.bn * k_slice / (per_cu_rate(c, operands) * 1e6);
    const double floor = std::ceil(per_cu / 2) * std::ceil(k_slice / mfma_tile_bk(i)) *
                         window_floor_us(operands);
    return std::fmax(work, floor) + c.t1_us + c.t0_us;
}

// Index into kTiles of the configuration the model prefers for this shape, and
// its modelled time in microseconds.
static int choose_tile(int M, int N, int K, int cus, double *model_us = nullptr) {
    int best = 0;
    double best_us = 0;
    for (int i = 0; i < kTileCount; ++i) {
        const double us = tile_us(i, M, N, K, cus);
        if (i == 0 || us < best_us) {
            best = i;
            best_us = us;
        }
    }
    if (model_us) *model_us = best_us;
    return best;
}

static hipError_t launch_layout(const Problem &p, hipStream_t s, int tile) {
    if (p.ta) return p.tb ? launch_mfma_tt(p, s, tile) : launch_mfma_tn(p, s, tile);
    return p.tb ? launch_mfma_nt(p, s, tile) : launch_mfma_nn(p, s, tile);
}

hipError_t launch_mfma(const Problem &p, hipStream_t s) {
    return launch_layout(p, s, choose_tile(p.M, p.N, p.K, compute_units()));
}

int mfma_tile_count() { return kTileCount; }

const char *mfma_tile_name(int tile) {
    return tile >= 0 && tile < kTileCount ? kTiles[tile].name : nullptr;
}

int mfma_select(int M, int N, int K, int cus) { return choose_tile(M, N, K, cus > 0 ? cus : 256); }

double mfma_model_us(int M, int N, int K, int cus) {
    double us = 0;
    choose_tile(M, N, K, cus > 0 ? cus : 256, &us);
    return us;
}

int mfma_tile_bk(int tile) {
    switch (tile) {
    case 0: return TileHuge::BK;
    case 1: return TileWide::BK;
    case 2: return TileSplit192::BK;
    case 3: return TileTall::BK;
    case 4: return TileSmall::BK;
    case 5: return TileSplit64::BK;
    case 6: return TileTiny::BK;
    case 7: return TileTiny64::BK;
    default: return 0;
    }
}

double mfma_model_tile_us(int tile, int M, int N, int K, int cus, int slices) {
    if (tile < 0 || tile >= kTileCount || slices < 1) return 1e30;
    return split_tile_us(tile, M, N, K, cus > 0 ? cus : 256, slices);
}

hipError_t launch_mfma_splitk(const Problem &p, hipStream_t s, int tile, int slices, float *ws) {
    if (p.ta) return p.tb ? launch_mfma_tt_splitk(p, s, tile, slices, ws)
                          : launch_mfma_tn_splitk(p, s, tile, slices, ws);
    return p.tb ? launch_mfma_nt_splitk(p, s, tile, slices, ws)
                : launch_mfma_nn_splitk(p, s, tile, slices, ws);
}

hipError_t launch_mfma_tile(const Problem &p, hipStream_t s, int tile) {
    if (tile < 0 || tile >= kTileCount) return hipErrorInvalidValue;
    return launch_layout(p, s, tile);
}

}  // namespace sgemm
