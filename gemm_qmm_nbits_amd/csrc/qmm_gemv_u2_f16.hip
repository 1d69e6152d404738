// Instantiation of the GEMV kernels for one weight format and activation type.
#include "qmm_gemv_impl.h"

namespace qmm {
template hipError_t launch_at_type<GEMV_AFFINE, 2, QMM_F16>(const GemvArgs& g, int R, hipStream_t st);
}  // namespace qmm
