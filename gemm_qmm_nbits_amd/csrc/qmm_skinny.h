// Interface of the skinny matrix-core path (qmm_skinny.hip) for the host runtime.
#pragma once

#include "qmm_internal.h"

namespace qmm {

// Skinny matrix-core path for 8 < M <= kSkinnyMaxM (blocks >= 32 codes): the same
// operands as the prefill path (A16 in the workspace, W16 = fp16 of the exact
// dequant), 16-row M tiles, one load and dequantization per weight.
constexpr int64_t kSkinnyMaxM = 64;
bool skinny_applies(int64_t M, int64_t N, int64_t Kp, int block, int64_t row_bytes, int64_t nblk);
hipError_t launch_skinny(const PrefillArgs& p, hipStream_t st);
// Reduction splits of the skinny path (a function of the shape only; at most the
// splits the workspace holds partial sums for).
int skinny_splits(int64_t M, int64_t N, int64_t Kp);
// Ragged multi-token MoE matmul: rows of X grouped by expert, u4 expert weights.
struct RaggedArgs {
  const uint16_t* X;  // fp16 [R][K], K % 8 == 0
  int64_t R, K, N, E;
  const int32_t* offsets;  // [E + 1]
  const uint8_t* W;        // [E][N][nblk][block / 2]
  const uint16_t* scales;  // fp16 [E][N][nblk]
  const uint8_t* zp;       // packed u4 [E][N][ceil(nblk / 2)] or NULL (8)
  const uint16_t* bias;    // fp16 [E][N] or NULL
  int block, block_log2;
  int64_t nblk, row_bytes, zp_row_bytes;
  uint16_t* Y;             // fp16 [R][N]
};
hipError_t launch_ragged(const RaggedArgs& p, hipStream_t st);

// C = (((P[0] + P[1]) + ...) + P[S-1]) * rs[row] + bias, in C's type (rs NULL: 1)
// (qmm_prefill.hip).
hipError_t launch_reduce_splits(const float* P, int S, int64_t M, int64_t N, int64_t ldc, const float* rs,
                                const void* bias, void* C, int c_type, hipStream_t st);

}  // namespace qmm
