// mfma_nn.hip -- matrix-core kernels for op(A) = A, op(B) = B.
#include "mfma_kernel.h"

namespace sgemm {

SGEMM_MFMA_LAUNCHER(launch_mfma_nn, false, false)

}  // namespace sgemm
