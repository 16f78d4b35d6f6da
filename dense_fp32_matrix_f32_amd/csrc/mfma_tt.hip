// mfma_tt.hip -- matrix-core kernels for op(A) = A transposed, op(B) = B transposed.
#include "mfma_kernel.h"

namespace sgemm {

SGEMM_MFMA_LAUNCHER(launch_mfma_tt, true, true)

}  // namespace sgemm
