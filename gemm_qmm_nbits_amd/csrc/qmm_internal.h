// Internal interfaces between the host runtime (qmm_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

enum { GEMV_AFFINE = 0, GEMV_CODEBOOK = 1 };

struct GemvArgs {
  const void* A;
  int a_type;
  int64_t M, K, N;
  const uint8_t* W;
  int64_t row_bytes;  // bytes per weight row = nblk * block * bits / 8
  int64_t nchunks;    // row_bytes / 16 (chunked kernel)
  int fmt;            // GEMV_AFFINE or GEMV_CODEBOOK
  int bits;
  int block;
  int block_log2;
  int64_t nblk;
  const uint16_t* scales;  // affine: fp16 [N][nblk]
  const float* absmax;     // codebook: fp32 [N][nblk]
  const float* codebook;   // codebook: fp32 [16]
  const void* zp;
  int zp_kind;
  float uniform_zp;
  int64_t zp_row_bytes;
  const void* bias;
  void* C;
  int c_type;
  int lpr_log2;  // lanes per row = 1 << lpr_log2 (fixed by K, block, bits)
  int a_vec;     // A rows allow 4-element vector loads (16-byte aligned base, K % 4 == 0)
  int chunked;   // use the chunked kernel (row_bytes % 16 == 0 and W 16-byte aligned)
  int mt;        // rows of A handled per kernel instance: 1, 2, 4 or 8 (>= M)
  int slice_chunks;  // chunks of A staged in LDS per K-slice (a multiple of 1 << lpr_log2)
  size_t lds_bytes;  // dynamic LDS of the chunked kernel
  int num_cus;       // compute units of the device
  int wg_per_cu;     // resident work-groups per compute unit used to size the grid
};

constexpr size_t kMaxGemvLds = 160 * 1024;   // LDS per work-group on gfx950
constexpr size_t kGemvLdsBudget = 96 * 1024; // preferred A staging size per work-group

// Fill mt, slice_chunks, lds_bytes, wg_per_cu (and clear `chunked` when no slice fits).
void gemv_plan(GemvArgs& g, int num_cus);

int gemv_lanes_per_row_log2(int64_t nchunks);
int gemv_row_lanes_log2(int64_t nchunks, int64_t N);
hipError_t launch_gemv(GemvArgs g, int rows_per_lane, hipStream_t st);

struct DequantArgs {
  const uint8_t* W;
  int fmt;
  int bits;
  int block;
  int64_t N, K, nblk, row_bytes;
  const uint16_t* scales;
  const float* absmax;
  const float* codebook;
  const void* zp;
  int zp_kind;
  float uniform_zp;
  int64_t zp_row_bytes;
  void* out;
  int out_type;
};
hipError_t launch_dequant(const DequantArgs& d, hipStream_t st);

hipError_t launch_uniform_check(const uint16_t* zp, int64_t count, uint32_t* scratch,
                                hipStream_t st);
constexpr int kUniformPartials = 256;

// A (fp32 / bf16) -> fp16, round to nearest even, count elements.
// dst[m][k] = fp16(src[m][k]) for k < K, 0 for K <= k < Kp (rows of Kp elements).
hipError_t launch_cast_pad_f16(const void* src, int src_type, int64_t M, int64_t K, int64_t Kp,
                               uint16_t* dst, hipStream_t st);

struct PrefillArgs {
  const uint16_t* A16;  // fp16 [M][Kp], k >= K zero
  int64_t M, N, K;
  int64_t Kp;   // K rounded up to a multiple of 64
  int64_t ldc;  // row stride of C (elements)
  const uint8_t* W;
  int bits, block, block_log2;
  int64_t nblk, row_bytes;
  int fmt;                 // GEMV_AFFINE or GEMV_CODEBOOK
  const uint16_t* scales;  // affine: fp16 [N][nblk]
  const float* absmax;     // codebook: fp32 [N][nblk]
  const float* codebook;   // codebook: fp32 [16]
  const void* zp;
  int zp_kind;
  float zconst;  // zero point for QMM_ZP_NONE / QMM_ZP_UNIFORM
  int64_t zp_row_bytes;
  const void* bias;
  void* C;
  int c_type;
  int ntiles, mtiles;
  int tiles_grid;   // work-groups per split (XCD-padded tile grid)
  int splits, spl;  // reduction splits and stages per split
  float* partials;  // fp32 [splits][M][ldc] workspace (splits > 1), or NULL
};
hipError_t launch_prefill(PrefillArgs p, hipStream_t st);
int prefill_splits(int64_t M, int64_t N, int64_t Kp);

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
// candidate: rows per lane (1 or 2), plus kQmoePerSlot for the per-slot form
constexpr int kQmoePerSlot = 16;
hipError_t launch_qmoe_fc1(const QmoeArgs& a, int candidate, hipStream_t st);
hipError_t launch_qmoe_fc2(const QmoeArgs& a, int candidate, hipStream_t st);

}  // namespace qmm
