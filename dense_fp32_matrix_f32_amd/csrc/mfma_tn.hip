// mfma_tn.hip -- matrix-core kernels for op(A) = A transposed, op(B) = B.
#include "mfma_kernel.h"

namespace sgemm {

SGEMM_MFMA_LAUNCHER(launch_mfma_tn, true, false)

}  // namespace sgemm
