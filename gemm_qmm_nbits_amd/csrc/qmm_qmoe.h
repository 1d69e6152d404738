// Internal interfaces between the host runtime (qmm_api.cpp) and the MoE decode
// kernels (qmm_qmoe.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

struct QmoeArgs {
  const uint16_t* X;
  int64_t T, H, I, E;
  int k;
  const int32_t* ids;
  const float* rw;
  qmoe_weights fc1, fc2;
  int block;
  int mode;
  int64_t fc1_row_bytes, fc1_nblk, fc1_zp_row_bytes, fc1_chunks;
  int fc1_lpr_log2;
  int64_t fc2_row_bytes, fc2_nblk, fc2_zp_row_bytes, fc2_chunks;
  int fc2_lpr_log2;
  uint16_t* h;      // scratch: fp16 [T][k][I]
  int8_t* xq_out;   // int8 mode: [T][H] codes of x (natural order)
  float* xs_out;    // int8 mode: [T][H/32] scales of x
  int8_t* hq_out;   // int8 mode: [T][k][I] codes of h
  float* hs_out;    // int8 mode: [T][k][I/32] scales of h
  uint16_t* Y;
  int num_cus;      // compute units of the device
  // single-launch form (fp mode): groups per wave per work item, items per slot,
  // fp32 slot sums [T*k][H] and the self-resetting sync words (see qmoe_sync_words)
  int f_gpw1, f_gpw2;
  int f_wpc;  // work-groups per compute unit in the grid (capped by occupancy)
  int64_t f_n1s, f_n2s;
  float* zpart;
  uint32_t* sync;
};
// Sync words of the single-launch form, in scratch: [0] next work item, [1] finished
// work-groups, [2] error flag (a wait that timed out), [3] unused, then the finished
// fc1 items of each slot [T*k], then the finished slots of each fc2 row tile [T][n2s].
// They must be zero before the first call on a scratch buffer; every call leaves them
// zero.
constexpr int kSyncHead = 4;
inline int64_t qmoe_sync_words(int64_t T, int64_t H, int k) {
  return kSyncHead + T * k + T * ((H + 3) / 4);
}
// Geometry of the single-launch form for candidate c: row groups per wave per work
// item kQmoeFusedGpw[c / 3], work-groups per compute unit kQmoeFusedWpc[c % 3]; false
// when the form does not apply (int8 mode, 32-bit offsets, LDS).
constexpr int kQmoeFusedGpw[] = {1, 2, 4};
constexpr int kQmoeFusedWpc[] = {1, 2, 4};
constexpr int kNumQmoeFused = 9;
bool qmoe_fused_plan(QmoeArgs& a, int candidate);
hipError_t launch_qmoe_fused(const QmoeArgs& a, hipStream_t st);
size_t qmoe_fc1_lds_bytes(const QmoeArgs& a);
size_t qmoe_fc2_lds_bytes(const QmoeArgs& a);
// candidate: rows per lane (1 or 2), plus kQmoePerSlot for the per-slot form, or
// kQmoeOnePerCu for the persistent form with one work-group per compute unit
constexpr int kQmoePerSlot = 16;
constexpr int kQmoeOnePerCu = 32;
hipError_t launch_qmoe_fc1(const QmoeArgs& a, int candidate, hipStream_t st);
hipError_t launch_qmoe_fc2(const QmoeArgs& a, int candidate, hipStream_t st);

}  // namespace qmm
