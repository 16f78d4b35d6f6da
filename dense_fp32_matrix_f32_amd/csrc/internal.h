// internal.h -- declarations shared by the kernel files and the C-ABI layer.
// Not installed; the public interface is include/sgemm_f32.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_order.h"

namespace sgemm {

// Validated arguments of one product C = A·B (row-major, element strides).
struct Problem {
    int M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
};

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

hipError_t launch_zero_fill(const Problem &p, hipStream_t s);
hipError_t launch_naive(const Problem &p, hipStream_t s);
hipError_t launch_lds_tiled(const Problem &p, hipStream_t s);
hipError_t launch_valu_regblock(const Problem &p, hipStream_t s);
hipError_t launch_mfma(const Problem &p, hipStream_t s);
// The MFMA rung with one tile configuration forced (0 <= tile < mfma_tile_count()).
hipError_t launch_mfma_tile(const Problem &p, hipStream_t s, int tile);
int mfma_tile_count();
const char *mfma_tile_name(int tile);
// The configuration launch_mfma() uses for this shape on `cus` compute units.
int mfma_select(int M, int N, int K, int cus);
hipError_t launch_skinny(const Problem &p, hipStream_t s);
hipError_t launch_skinny_n(const Problem &p, hipStream_t s);

}  // namespace sgemm
