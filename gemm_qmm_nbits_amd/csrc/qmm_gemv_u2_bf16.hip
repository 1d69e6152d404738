// Instantiation of the integer-plane GEMV for 2-bit affine weights and bf16 activations.
#include "qmm_gemv_stream.h"

namespace qmm {
template hipError_t launch_ip_at_type<2, QMM_BF16>(const GemvArgs& g, int R, hipStream_t st);
}  // namespace qmm
