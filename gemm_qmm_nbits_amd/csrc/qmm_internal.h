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

}  // namespace qmm
