// mfma_nt.hip -- matrix-core kernels for op(A) = A, op(B) = B transposed.
#include "mfma_kernel.h"

namespace sgemm {

SGEMM_MFMA_LAUNCHER(launch_mfma_nt, false, true)

}  // namespace sgemm
