// Internal interfaces between the host runtime (qmm_api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

// Launch timing, a measurement aid: while the calling host thread has it switched on
// (qmm_launch_timing_begin), each kernel the library launches from that thread records
// the start and the end of its execution on the device into the next pair of a fixed
// set of HIP events; launches past the set, and every launch while it is off, go out
// as plain launches.
struct LaunchTiming {
  int on = 0;
  int next = 0;
  int cap = 0;
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
};
inline thread_local LaunchTiming g_launch_timing;

// Every kernel launch of the library goes through here.
template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args... args) {
  LaunchTiming& t = g_launch_timing;
  if (t.on && t.next < t.cap) {
    const int i = t.next++;
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, t.start[i], t.stop[i], 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  }
}

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
// rows_per_lane above kGemvMxBase selects the matrix-core form of the 2-bit GEMV with
// rows_per_lane - kGemvMxBase groups of 16 rows per wave (where the shape suits it;
// elsewhere the v_dot8 kernel with 2 rows per lane, which gives the same bits).
constexpr int kGemvMxBase = 16;
hipError_t launch_gemv(GemvArgs g, int rows_per_lane, hipStream_t st);
// Whether the matrix-core form serves this planned shape.
bool gemv_mx_supported(const GemvArgs& g);

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
hipError_t launch_nested_absmax(const uint8_t* codes, const float* table, const float* scales, float offset,
                                int group, int64_t count, float* out, hipStream_t st);
constexpr int kUniformPartials = 256;

// A (fp32 / fp16 / bf16) -> fp16 rows of Kp elements with a per-row power-of-two
// pre-scale: dst[m][k] = fp16(src[m][k] * 2^s_m) for k < K, 0 for K <= k < Kp, and
// row_scale[m] = 2^-s_m (s_m puts the row's largest magnitude in [2^14, 2^15); 0 for
// fp16 sources, zero rows and rows with a non-finite value).
hipError_t launch_cast_pad_f16(const void* src, int src_type, int64_t M, int64_t K, int64_t Kp,
                               uint16_t* dst, float* row_scale, hipStream_t st);

// A zero point z for which fp32((q - z) * s) == fma(q, s, -(z * s)) for every code q
// in 0..255 (or -128..127) and every fp16 scale s: q - z is exact in fp32 (|z| < 2^8,
// lowest set bit at 2^-15 or above) and z * s is exact (z has at most 13 significant
// bits, s has 11), so the one rounding of the fma is the rounding of the product.
inline bool zconst_fma_exact(float z) {
  if (!(z > -256.0f && z < 256.0f)) return false;
  const float t = z * 32768.0f;  // exact: a power of two
  if (t != (float)(int32_t)t) return false;
  uint32_t u = (uint32_t)(t < 0 ? -t : t);
  if (u == 0) return true;
  while (!(u & 1u)) u >>= 1;
  return u < (1u << 13);
}

struct PrefillArgs {
  const uint16_t* A16;  // fp16 [M][lda]: the cast workspace (lda = Kp, k >= K zero) or fp16 A itself
  const float* row_scale;  // [M] factor of each row's sums (the cast's 2^-s_m), or NULL for 1
  int64_t lda;  // row stride of A16 in elements (Kp, or K for fp16 A read in place)
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
  int zconst_fma;  // zconst_fma_exact(zconst): the dequantization may use one fma per code
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

// Streaming read of `bytes` (a multiple of 16) by `groups` work-groups (qmm_probe.hip).
hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, int groups, hipStream_t st);

// Activation quantization ops (qmm_qdq.hip); arguments checked by the caller.
using QdqParams = qmm_qparams;
hipError_t launch_quantize_linear(const void* x, int x_type, int64_t n, QdqParams q, int bits, void* codes,
                                  hipStream_t st);
hipError_t launch_dequantize_linear(const void* codes, int64_t n, QdqParams q, int bits, void* y, int y_type,
                                    hipStream_t st);
hipError_t launch_fake_quantize(const void* x, int x_type, int64_t n, QdqParams q, int bits, void* y,
                                hipStream_t st);
hipError_t launch_qsigmoid(const void* in, int64_t n, QdqParams qi, QdqParams qo, int bits, void* out,
                           hipStream_t st);
hipError_t launch_qmul(const void* a, QdqParams qa, const void* b, QdqParams qb, int64_t n, QdqParams qc, int bits,
                       void* c, hipStream_t st);
hipError_t launch_qswiglu(const void* gate, const void* up, int x_type, int64_t n, int bits, const QdqParams* q,
                          void* y, hipStream_t st);

}  // namespace qmm
