// Instantiation of the codebook GEMV kernels for one activation type.
#include "qmm_gemv_cb_stream.h"

namespace qmm {
template hipError_t launch_cb_at_type<QMM_F32>(const GemvArgs& g, int R, hipStream_t st);
}  // namespace qmm
