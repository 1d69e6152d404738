// The MoE decode for callers that cannot allocate (code under stream capture, tight
// serving loops, harnesses that forbid hipMalloc): qmoe_decode_fused with its scratch
// in a static device array instead of a caller buffer.
//
// The array lives in this library's code object, one copy per device, for the life of
// the process.  Host code never uses its name as an address: the device address of
// the current device's copy is taken once per device with hipGetSymbolAddress and
// passed to the kernels like a caller's scratch.  The call never times tiling
// candidates (it uses the shape's cached choice, made by an earlier
// qmoe_decode_fused call, or the default tiling), so it calls no allocating routine.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qmm.h"
#include "qmm_qmoe.h"

namespace {

// sync words of the single-launch form sit in it and start at zero (static storage);
// every completed call leaves them at zero again
static __device__ __align__(256) uint8_t scratch[QMOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of this device's copy of `scratch`, looked up once per device.
qmm_status device_scratch(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (qmm_status)e;
  if (dev < 0 || dev >= kMaxDevices) return QMM_E_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return e != hipSuccess ? (qmm_status)e : QMM_E_DEVICE;
    addr[dev] = p;
  }
  *out = addr[dev];
  return QMM_OK;
}

}  // namespace

extern "C" qmm_status qmoe_decode_fused_noalloc(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E,
                                                int k, const int32_t* expert_ids, const float* expert_w,
                                                qmoe_weights fc1, qmoe_weights fc2, int bits, int block, int mode,
                                                uint16_t* Y, void* stream) {
  (void)hipGetLastError();
  void* sc = nullptr;
  const qmm_status s = device_scratch(&sc);
  if (s != QMM_OK) return s;
  // a shape whose scratch exceeds the array is refused (QMM_E_WORKSPACE) by the checks
  return qmm::qmoe_decode_run(X, T, H, I, E, k, expert_ids, expert_w, fc1, fc2, bits, block, mode, Y, sc,
                              QMOE_NOALLOC_SCRATCH_BYTES, stream, false);
}
