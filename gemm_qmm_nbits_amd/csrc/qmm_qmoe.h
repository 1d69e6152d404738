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
  // single-launch form: fc2 rows per lane, work-groups per compute unit, and the
  // self-resetting sync words in scratch (kQmoeSyncWords)
  int f_r2;
  int f_wpc;
  uint32_t* sync;
};
// Sync words of the single-launch form, at offset 0 of scratch, in slots of 256 bytes:
// slot 0 holds [0] the top arrival count (slots complete), [1] unused, [2] the error
// flag (a wait that timed out), [3] unused; slots 1 .. kQmoeSyncSubs hold [0] a
// sub-counter (work-groups b with b % kQmoeSyncSubs == slot - 1 arrived) and [1] a
// copy of the phase (flipped once per call by the last arrival).  All must be zero
// before the first call on a scratch buffer; every call leaves the counters zero and
// the phases equal, at 0 or 1.
constexpr int kQmoeSyncSubs = 32;
constexpr int kQmoeSyncSlotWords = 64;
constexpr int64_t kQmoeSyncWords = (1 + kQmoeSyncSubs) * kQmoeSyncSlotWords;
// Single-launch candidates: candidate c runs fc2 with kQmoeFusedR2[c % 2] rows per lane
// and kQmoeFusedWpc[c / 2] work-groups per compute unit (fewer when they do not fit).
constexpr int kQmoeFusedR2[] = {1, 2};
constexpr int kQmoeFusedWpc[] = {1, 2};
constexpr int kNumQmoeFused = 4;
// Fill the candidate's parameters; false when the shape does not suit it (LDS, 32-bit
// offsets).
bool qmoe_fused_plan(QmoeArgs& a, int candidate);
// hipErrorNotSupported when the shape does not fit the form (LDS, 32-bit offsets).
hipError_t launch_qmoe_fused(const QmoeArgs& a, hipStream_t st);
size_t qmoe_fc1_lds_bytes(const QmoeArgs& a);
size_t qmoe_fc2_lds_bytes(const QmoeArgs& a);
// candidate: rows per lane (1 or 2), plus kQmoePerSlot for the per-slot form,
// kQmoeOnePerCu for the persistent form with one work-group per compute unit, or
// kQmoeDedupe (below)
constexpr int kQmoePerSlot = 16;
constexpr int kQmoeOnePerCu = 32;
// fc1: each expert's rows read once per call for all its slots (fp mode, 1 < T <= 8);
// otherwise, and for fc2, the persistent form with the same rows per lane
constexpr int kQmoeDedupe = 64;
hipError_t launch_qmoe_fc1(const QmoeArgs& a, int candidate, hipStream_t st);
hipError_t launch_qmoe_fc2(const QmoeArgs& a, int candidate, hipStream_t st);

// The whole MoE decode call (checks, tiling choice, launches) on a given scratch
// buffer; may_time = false never times candidates (and so never allocates).
qmm_status qmoe_decode_run(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E, int k,
                           const int32_t* expert_ids, const float* expert_w, qmoe_weights fc1, qmoe_weights fc2,
                           int bits, int block, int mode, uint16_t* Y, void* scratch, size_t scratch_bytes,
                           void* stream, bool may_time);

}  // namespace qmm
