// internal.h -- declarations shared by the kernel files and the C-ABI layer.
// Not installed; the public interface is include/sgemm_f32.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_order.h"

namespace sgemm {

// Validated arguments of one product C = alpha*op(A)*op(B) + beta*C (row-major,
// element strides).  op(A) is A (M x K) or, with ta, the transpose of the K x M
// array A; op(B) is B (K x N) or, with tb, the transpose of the N x K array B.
// beta == 0 means C is not read.
struct Problem {
    int M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
    bool ta = false, tb = false;
    float alpha = 1.0f, beta = 0.0f;
};

// alpha*acc, plus beta*C when beta != 0 (C is not read otherwise).
__device__ __forceinline__ float epilogue(float acc, float alpha, float beta, const float *c) {
    return beta == 0.0f ? alpha * acc : fmaf(beta, *c, alpha * acc);
}

// hipLaunchKernel with typed arguments; returns the launch status itself
// rather than a sticky per-thread error.
template <typename... Params, typename... Args>
inline hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds_bytes,
                         hipStream_t stream, Args... args) {
    static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
    auto pack = [&](Params... p) {
        void *argv[] = {(void *)&p...};
        return hipLaunchKernel((const void *)kernel, grid, block, argv, lds_bytes, stream);
    };
    return pack(static_cast<Params>(args)...);
}

// C = beta*C without a product (alpha == 0 or K == 0); beta == 0 writes zeros.
hipError_t launch_scale(const Problem &p, hipStream_t s);
hipError_t launch_naive(const Problem &p, hipStream_t s);
hipError_t launch_lds_tiled(const Problem &p, hipStream_t s);
hipError_t launch_valu_regblock(const Problem &p, hipStream_t s);
hipError_t launch_mfma(const Problem &p, hipStream_t s);
// The MFMA rung with one tile configuration forced (0 <= tile < mfma_tile_count()).
hipError_t launch_mfma_tile(const Problem &p, hipStream_t s, int tile);
int mfma_tile_count();
const char *mfma_tile_name(int tile);
// The configuration launch_mfma() uses for this shape on `cus` compute units,
// and the cost model's time for it in microseconds.
int mfma_select(int M, int N, int K, int cus);
double mfma_model_us(int M, int N, int K, int cus);
// Compute units of the current device (256 if the query fails).
int compute_units();
// The fp32 product on the bf16 matrix cores with three-part operand splitting
// (untransposed operands only).
hipError_t launch_split(const Problem &p, hipStream_t s);
// Streaming kernels for products with few rows of C (any number of rows, in
// passes of 8): launch_skinny_rows (skinny.hip) when B is not transposed,
// launch_skinny_rows_tb (skinny_n.hip, on C^T = B^T * op(A)^T) when it is; and
// with few columns of C (passes of 8): launch_skinny_cols (skinny_n.hip) when A
// is not transposed, launch_skinny_cols_ta (skinny.hip, on C^T) when it is.
hipError_t launch_skinny_rows(const Problem &p, hipStream_t s);
hipError_t launch_skinny_rows_tb(const Problem &p, hipStream_t s);
hipError_t launch_skinny_cols(const Problem &p, hipStream_t s);
hipError_t launch_skinny_cols_ta(const Problem &p, hipStream_t s);
// Split-k: `slices` unscaled partial products of op(A)*op(B) go to the workspace
// planes ws[q*M*N + i*N + j], then launch_splitk_reduce() forms
// C = alpha * (sum over q) + beta * C, adding the planes in an order fixed by
// (M, N, slices).  launch_mfma_splitk() takes the
// configurations TileWide (1), TileSmall (4) and TileSplit64 (5).
hipError_t launch_mfma_splitk(const Problem &p, hipStream_t s, int tile, int slices, float *ws);
hipError_t launch_splitk_reduce(const Problem &p, int slices, const float *ws, hipStream_t s);
// Modelled time (microseconds) of the product kernel of configuration `tile` on
// `cus` CUs when the k windows are split into `slices` slices (products only,
// not the reduction).
double mfma_model_tile_us(int tile, int M, int N, int K, int cus, int slices);
// k window of configuration `tile` (0 for an unknown id).
int mfma_tile_bk(int tile);

}  // namespace sgemm
