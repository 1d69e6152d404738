// Instantiation of the integer-plane GEMV (v_dot8 and matrix-core forms) for 2-bit affine weights and f32 activations.
#include "qmm_gemv_mx.h"
#include "qmm_gemv_stream.h"

namespace qmm {
template hipError_t launch_ip_at_type<2, QMM_F32>(const GemvArgs& g, int R, hipStream_t st);
template hipError_t launch_mx_at_type<QMM_F32>(const GemvArgs& g, int R, hipStream_t st);
}  // namespace qmm
