// Measurement helper: the HBM read rate a plain streaming kernel reaches on this device,
// the practical ceiling next to the spec peak for the weight-streaming kernels.
//
// Every 16-byte piece of the buffer is read once with a 128-bit load; work-group g reads
// the contiguous range [g * span, (g + 1) * span) with its lanes on consecutive pieces,
// four loads in flight per lane.  The xor of everything read goes to one word per
// work-group, so no load can be dropped.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const uint4* buf, int64_t pieces,
                                                                 int64_t span, uint32_t* sink) {
  const int64_t begin = (int64_t)blockIdx.x * span;
  const int64_t end = begin + span < pieces ? begin + span : pieces;
  uint32_t x = 0;
  int64_t i = begin + threadIdx.x;
  for (; i + 3 * kProbeThreads < end; i += 4 * kProbeThreads) {
    const uint4 a = buf[i], b = buf[i + kProbeThreads], c = buf[i + 2 * kProbeThreads],
                d = buf[i + 3 * kProbeThreads];
    x ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < end; i += kProbeThreads) {
    const uint4 a = buf[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  x ^= __shfl_xor(x, 1, 64);
  x ^= __shfl_xor(x, 2, 64);
  x ^= __shfl_xor(x, 4, 64);
  x ^= __shfl_xor(x, 8, 64);
  x ^= __shfl_xor(x, 16, 64);
  x ^= __shfl_xor(x, 32, 64);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) r ^= part[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, int groups, hipStream_t st) {
  const int64_t pieces = bytes / 16;
  const int64_t span = (pieces + groups - 1) / groups;
  launch(hbm_read_kernel, dim3((unsigned)groups), dim3(kProbeThreads), 0, st, (const uint4*)buf, pieces,
                     span, sink);
  return hipSuccess;
}

}  // namespace qmm
