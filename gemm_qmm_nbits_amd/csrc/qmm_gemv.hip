// Dispatch of the weight-streaming GEMV kernels (instantiated in qmm_gemv_*.hip).
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_gemv_mx.h"

namespace qmm {

template <int AT>
hipError_t launch_cb_at_type(const GemvArgs& g, int R, hipStream_t st);
template <int BITS, int AT>
hipError_t launch_ip_at_type(const GemvArgs& g, int R, hipStream_t st);
template <int FMT, int BITS, int AT>
hipError_t launch_at_type(const GemvArgs& g, int R, hipStream_t st);
template <int AT>
hipError_t launch_mx_at_type(const GemvArgs& g, int R, hipStream_t st);

// 3-bit and signed 8-bit affine weights: the fp32 kernel (codes decoded to fp32)
template <int BITS>
static hipError_t launch_affine_fp32(const GemvArgs& g, int R, hipStream_t st) {
  switch (g.a_type) {
    case QMM_F32: return launch_at_type<GEMV_AFFINE, BITS, QMM_F32>(g, R, st);
    case QMM_F16: return launch_at_type<GEMV_AFFINE, BITS, QMM_F16>(g, R, st);
    default: return launch_at_type<GEMV_AFFINE, BITS, QMM_BF16>(g, R, st);
  }
}

// codebook weights: fp32 kernels with the LDS centroid table
static hipError_t launch_codebook(const GemvArgs& g, int R, hipStream_t st) {
  switch (g.a_type) {
    case QMM_F32: return launch_cb_at_type<QMM_F32>(g, R, st);
    case QMM_F16: return launch_cb_at_type<QMM_F16>(g, R, st);
    default: return launch_cb_at_type<QMM_BF16>(g, R, st);
  }
}

// affine weights: integer-plane kernel
template <int BITS>
static hipError_t launch_affine(const GemvArgs& g, int R, hipStream_t st) {
  switch (g.a_type) {
    case QMM_F32: return launch_ip_at_type<BITS, QMM_F32>(g, R, st);
    case QMM_F16: return launch_ip_at_type<BITS, QMM_F16>(g, R, st);
    default: return launch_ip_at_type<BITS, QMM_BF16>(g, R, st);
  }
}

// 2-bit affine weights at M = 1: matrix-core form (hipErrorNotSupported where the
// shape does not suit it)
static hipError_t launch_affine_mx(const GemvArgs& g, int R, hipStream_t st) {
  switch (g.a_type) {
    case QMM_F32: return launch_mx_at_type<QMM_F32>(g, R, st);
    case QMM_F16: return launch_mx_at_type<QMM_F16>(g, R, st);
    default: return launch_mx_at_type<QMM_BF16>(g, R, st);
  }
}

bool gemv_mx_supported(const GemvArgs& g) { return gemv_mx_pairs(g) > 0 && ((uintptr_t)g.scales & 15u) == 0; }

// Generic path for layouts the chunked kernel cannot read (row length not a
// multiple of 16 bytes, or unaligned pointers): one wave per output column n,
// lane l handles codes k = l, l+64, ..., each dequantized exactly as defined.
__global__ __launch_bounds__(256) void gemv_generic_kernel(GemvArgs g) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= g.N) return;
  float acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = 0.0f;
  const int bits = g.fmt == GEMV_CODEBOOK ? 4 : g.bits;
  const int blob = g.block * bits / 8;   // bytes per block
  for (int64_t k = lane; k < g.K; k += 64) {
    const int b = (int)(k / g.block);
    const int j = (int)(k % g.block);
    const int32_t q = code_at(g.W + n * g.row_bytes + (int64_t)b * blob, j, bits);
    float w;
    if (g.fmt == GEMV_CODEBOOK) {
      w = __fmul_rn(g.codebook[q], g.absmax[n * g.nblk + b]);
    } else {
      const float s = f16_to_f32(g.scales[n * g.nblk + b]);
      const float z = zero_point(g.zp, g.zp_kind, g.uniform_zp, bits, n, b, g.zp_row_bytes, g.nblk);
      w = dequant_affine(q, z, s);
    }
    for (int m = 0; m < 8; ++m)
      if (m < g.M) acc[m] = fmaf(load_elem_rt(g.A, g.a_type, (int64_t)m * g.K + k), w, acc[m]);
  }
  for (int m = 0; m < 8; ++m) acc[m] = group_sum(acc[m], 64);
  if (lane == 0) {
    const float bv = g.bias ? load_elem_rt(g.bias, g.c_type, n) : 0.0f;
    for (int m = 0; m < 8; ++m)
      if (m < g.M) store_elem_rt(g.C, g.c_type, (int64_t)m * g.N + n, acc[m] + bv);
  }
}


int gemv_lanes_per_row_log2(int64_t nchunks) {
  // Widest row group (fewest sequential chunks per lane) that keeps at least 80%
  // of the lane slots busy; otherwise the group with the fewest idle slots
  // (ties to the wider one).  Depends on the chunk count only.
  for (int l = 6; l >= 3; --l) {
    const int64_t lpr = 1LL << l;
    const int64_t slots = ((nchunks + lpr - 1) / lpr) * lpr;
    if (nchunks * 5 >= slots * 4) return l;
  }
  int best = 6;
  int64_t best_slots = ((nchunks + 63) / 64) * 64;
  for (int l = 5; l >= 3; --l) {
    const int64_t lpr = 1LL << l;
    const int64_t slots = ((nchunks + lpr - 1) / lpr) * lpr;
    if (slots < best_slots) {
      best_slots = slots;
      best = l;
    }
  }
  return best;
}

int gemv_row_lanes_log2(int64_t nchunks, int64_t N) {
  // Lanes per row for the GEMV: the group width with the best product of lane
  // efficiency (busy lane slots / all slots of a row) and parallelism (row tiles of
  // one 8-wave work-group, relative to a fixed 512), ties to the wider group.  A
  // function of the shape only, so every device and every tiling candidate use the
  // same summation order.
  int best = 6;
  double best_score = -1.0;
  for (int l = 6; l >= 3; --l) {
    const int64_t lpr = 1LL << l;
    const int64_t slots = ((nchunks + lpr - 1) / lpr) * lpr;
    const double eff = slots > 0 ? (double)nchunks / (double)slots : 0.0;
    const int64_t rows_per_tile = 8 * (64 / lpr);
    const int64_t tiles = (N + rows_per_tile - 1) / rows_per_tile;
#ifndef QMM_LPR_TARGET
#define QMM_LPR_TARGET 512
#endif
    const double par = tiles >= QMM_LPR_TARGET ? 1.0 : (double)tiles / (double)QMM_LPR_TARGET;
    const double score = eff * par;
    if (score > best_score + 1e-12) {
      best_score = score;
      best = l;
    }
  }
  return best;
}

void gemv_plan(GemvArgs& g, int num_cus) {
  g.mt = g.M <= 1 ? 1 : g.M <= 2 ? 2 : g.M <= 4 ? 4 : 8;
  g.num_cus = num_cus > 0 ? num_cus : 256;
  // LDS bytes per chunk slot per A row: codebook kernel = fp32 activations (WPC + 4
  // floats) + 4 group sums; integer-plane kernel = the planes (12 or 6 words per
  // weight dword, 4 words of padding) + 4 group records of four words
  int64_t cs_bytes;
  if (g.fmt == GEMV_CODEBOOK) cs_bytes = (int64_t)(32 + 4) * 4 + 4 * 4;
  else if (g.bits == 3) cs_bytes = (int64_t)(32 + 4) * 4 + 4 * 4;   // fp32 kernel, 32 codes per chunk
  else if (g.bits == 8) cs_bytes = (int64_t)(16 + 4) * 4 + 4 * 4;   // fp32 kernel, 16 codes per chunk
  else if (g.bits == 2) cs_bytes = (int64_t)(4 * 12 + 4) * 4 + 4 * 16;
  else cs_bytes = (int64_t)(4 * 6 + 4) * 4 + 4 * 16;
  const int64_t lpr = 1LL << g.lpr_log2;
  const int64_t per_iter = (int64_t)g.mt * lpr * cs_bytes;  // one chunk per lane, all A rows
  const int64_t iters_all = (g.nchunks + lpr - 1) / lpr;
  int64_t iters = (int64_t)kGemvLdsBudget / per_iter;
  if (iters < 1) iters = 1;
  if (iters > iters_all) iters = iters_all > 0 ? iters_all : 1;
  g.slice_chunks = (int)(iters * lpr);
  // A slice + group records + 16 floats (the codebook kernel's table, the integer-plane
  // kernels' trash line); the kernel adds its output buffer
  g.lds_bytes = (size_t)(iters * per_iter) + 16 * sizeof(float);
  const size_t total = g.lds_bytes + 4096 * sizeof(float);
  if (total > kMaxGemvLds) {
    g.chunked = 0;  // no slice fits: generic kernel
    g.lds_bytes = 0;
  }
  int per_cu = g.lds_bytes ? (int)(kMaxGemvLds / total) : 2;
  if (per_cu > 3) per_cu = 3;
  if (per_cu < 1) per_cu = 1;
  g.wg_per_cu = per_cu;
}

hipError_t launch_gemv(GemvArgs g, int rows_per_lane, hipStream_t st) {
  if (!g.chunked) {
    const dim3 grid((unsigned)((g.N + 3) / 4));
    launch(gemv_generic_kernel, grid, dim3(256), 0, st, g);
    return hipSuccess;
  }
  if (rows_per_lane > kGemvMxBase) {
    const hipError_t e = gemv_mx_supported(g) ? launch_affine_mx(g, rows_per_lane - kGemvMxBase, st)
                                              : hipErrorNotSupported;
    if (e != hipErrorNotSupported) return e;
    rows_per_lane = 2;
  }
  if (g.fmt == GEMV_CODEBOOK) return launch_codebook(g, rows_per_lane, st);
  if (g.bits == 2) return launch_affine<2>(g, rows_per_lane, st);
  if (g.bits == 3) return launch_affine_fp32<3>(g, rows_per_lane, st);
  if (g.bits == 8) return launch_affine_fp32<8>(g, rows_per_lane, st);
  return launch_affine<4>(g, rows_per_lane, st);
}

}  // namespace qmm
