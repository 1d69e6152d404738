// Instantiation of the fp32 GEMV for 3-bit and signed 8-bit affine weights and bf16 activations.
#include "qmm_gemv_impl.h"

namespace qmm {
template hipError_t launch_at_type<GEMV_AFFINE, 3, QMM_BF16>(const GemvArgs& g, int R, hipStream_t st);
template hipError_t launch_at_type<GEMV_AFFINE, 8, QMM_BF16>(const GemvArgs& g, int R, hipStream_t st);
}  // namespace qmm
