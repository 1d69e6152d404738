// Small kernels: bit-exact dequantization, uniform zero-point detection, A cast.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// ---- dense dequantization --------------------------------------------------
// out[n][k] = fp32(fp32(q - zp) * s)  (affine, [P1] "What", commit 1)
//           = fp32(codebook[q] * absmax) (codebook, [P3] "Summary")
// fp16 output is the round-to-nearest-even of that fp32 value.
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs d) {
  const int64_t total = d.N * d.K;
  const int blob = d.block * d.bits / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / d.K;
    const int64_t k = i - n * d.K;
    const int b = (int)(k / d.block);
    const int j = (int)(k - (int64_t)b * d.block);
    const int32_t q = code_at(d.W + n * d.row_bytes + (int64_t)b * blob, j, d.bits);
    float w;
    if (d.fmt == GEMV_CODEBOOK) {
      w = __fmul_rn(d.codebook[q], d.absmax[n * d.nblk + b]);
    } else {
      const float s = f16_to_f32(d.scales[n * d.nblk + b]);
      const float z = zero_point(d.zp, d.zp_kind, d.uniform_zp, d.bits, n, b, d.zp_row_bytes, d.nblk);
      w = dequant_affine(q, z, s);
    }
    if (d.out_type == QMM_F16) ((uint16_t*)d.out)[i] = f32_to_f16(materialize(w));
    else ((float*)d.out)[i] = w;
  }
}

hipError_t launch_dequant(const DequantArgs& d, hipStream_t st) {
  const int64_t total = d.N * d.K;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  launch(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, d);
  return hipSuccess;
}

// ---- nested absmax ([P3] "Testing plan": nested absmax) ------------------------
// out[i] = fp32(fp32(table[codes[i]] * scales[i / group]) + offset), each operation
// rounded once (no contraction).
__global__ __launch_bounds__(256) void nested_absmax_kernel(const uint8_t* codes, const float* table,
                                                            const float* scales, float offset, int group,
                                                            int64_t count, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float prod = __fmul_rn(table[codes[i]], scales[i / group]);
    out[i] = __fadd_rn(materialize(prod), offset);
  }
}

hipError_t launch_nested_absmax(const uint8_t* codes, const float* table, const float* scales, float offset,
                                int group, int64_t count, float* out, hipStream_t st) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  launch(nested_absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, table, scales, offset,
                     group, count, out);
  return hipSuccess;
}

// ---- uniform zero point ([P1] "What", commit 1) ------------------------------
// Pass 1: partial p of kUniformPartials records whether its slice holds any fp16
// bit pattern different from zp[0].  Pass 2: one work-group folds the partials
// and writes {is_uniform, value bits}.  No atomics; deterministic.
__global__ __launch_bounds__(256) void uniform_partial_kernel(const uint16_t* zp, int64_t count,
                                                              uint32_t* partial) {
  const uint16_t first = zp[0];
  int diff = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    diff |= (zp[i] != first);
  diff = __syncthreads_or(diff);
  if (threadIdx.x == 0) partial[blockIdx.x] = (uint32_t)diff;
}

__global__ __launch_bounds__(256) void uniform_final_kernel(const uint16_t* zp, const uint32_t* partial,
                                                            uint32_t* result) {
  int diff = 0;
  for (int i = threadIdx.x; i < kUniformPartials; i += blockDim.x) diff |= (partial[i] != 0u);
  diff = __syncthreads_or(diff);
  if (threadIdx.x == 0) {
    const uint16_t first = zp[0];
    const bool is_nan = ((first & 0x7c00u) == 0x7c00u) && ((first & 0x03ffu) != 0u);
    const float v = f16_to_f32(first);
    result[0] = (!diff && !is_nan) ? 1u : 0u;
    result[1] = __float_as_uint(v);
  }
}

hipError_t launch_uniform_check(const uint16_t* zp, int64_t count, uint32_t* scratch,
                                hipStream_t st) {
  launch(uniform_partial_kernel, dim3(kUniformPartials), dim3(256), 0, st, zp, count,
                     scratch + 2);
  launch(uniform_final_kernel, dim3(1), dim3(256), 0, st, zp, scratch + 2, scratch);
  return hipSuccess;
}

// ---- A cast to fp16 (matrix-core paths; [P1] "What", commit 1: cast A once) -----
//
// Row m of A becomes dst[m][0..Kp) = fp16(a[m][k] * 2^s_m) for k < K and 0 past K,
// and rs[m] = 2^-s_m, the factor the epilogues apply to the row's sums.  The shift
// puts the row's largest magnitude |a| = f * 2^E (f in [0.5, 1)) into [2^14, 2^15):
// s_m = min(15 - E, 126), so no value overflows fp16 and small values keep their bits
// (both scalings are exact powers of two).  A row that is all zero or whose largest
// magnitude is not finite, and every row of fp16 activations (already in range), get
// s_m = 0.  One work-group of 256 threads per row; each thread holds its 8-element
// pieces in registers between the maximum and the conversion, so the row is read
// once (rows longer than 256 * 8 * kCastPieces elements are read twice).
constexpr int kCastThreads = 256;
constexpr int kCastPieces = 16;

__device__ __forceinline__ float cast_block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kCastThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ int cast_shift(float mx, int src_type) {
  if (src_type == QMM_F16 || !(mx <= 3.402823466e38f) || mx == 0.0f) return 0;
  int E = 0;
  (void)frexpf(mx, &E);
  const int s = 15 - E;
  return s < 126 ? s : 126;
}

// 8 consecutive elements of row m starting at k (k < K); VEC: K % 8 == 0 and a
// 16-byte aligned source, so the 8 lie in the row and come as aligned vectors.
template <int AT, bool VEC>
__device__ __forceinline__ void cast_load8(const void* src, int64_t m, int64_t K, int64_t k, float (&v)[8]) {
  const int64_t base = m * K + k;
  if constexpr (VEC) {
    if constexpr (AT == QMM_F32) {
      const f32x4* p = (const f32x4*)((const float*)src + base);
      const f32x4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 u = *(const uint4*)((const uint16_t*)src + base);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t lo = (uint16_t)(w[e] & 0xffffu), hi = (uint16_t)(w[e] >> 16);
        v[2 * e] = AT == QMM_F16 ? f16_to_f32(lo) : bf16_to_f32(lo);
        v[2 * e + 1] = AT == QMM_F16 ? f16_to_f32(hi) : bf16_to_f32(hi);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (k + e < K) ? load_elem<AT>(src, base + e) : 0.0f;
  }
}

__device__ __forceinline__ uint4 cast_store8(const float (&v)[8], int s) {
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = (uint32_t)f32_to_f16(ldexpf(v[2 * e], s)) | ((uint32_t)f32_to_f16(ldexpf(v[2 * e + 1], s)) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// CACHED: the row's pieces fit in registers (Kp <= 256 * 8 * kCastPieces).
template <int AT, bool VEC, bool CACHED>
__global__ __launch_bounds__(kCastThreads) void cast_rows_f16_kernel(const void* src, int64_t M, int64_t K,
                                                                    int64_t Kp, uint16_t* dst, float* rs) {
  __shared__ float red[kCastThreads / 64];
  const int64_t m = blockIdx.x;
  const int64_t pieces = Kp / 8;   // destination pieces of 8 elements
  const int64_t src_pieces = (K + 7) / 8;
  uint4* drow = (uint4*)(dst + m * Kp);
  float mx = 0.0f;
  if constexpr (CACHED) {
    float v[kCastPieces][8];
#pragma unroll
    for (int j = 0; j < kCastPieces; ++j) {
      const int64_t c = threadIdx.x + (int64_t)j * kCastThreads;
      if (c < src_pieces) cast_load8<AT, VEC>(src, m, K, c * 8, v[j]);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[j][e]));
    }
    const int s = cast_shift(cast_block_max(mx, red), AT);
#pragma unroll
    for (int j = 0; j < kCastPieces; ++j) {
      const int64_t c = threadIdx.x + (int64_t)j * kCastThreads;
      if (c < pieces) drow[c] = cast_store8(v[j], s);
    }
    if (threadIdx.x == 0) rs[m] = ldexpf(1.0f, -s);
  } else {
    for (int64_t c = threadIdx.x; c < src_pieces; c += kCastThreads) {
      float v[8];
      cast_load8<AT, VEC>(src, m, K, c * 8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
    }
    const int s = cast_shift(cast_block_max(mx, red), AT);
    for (int64_t c = threadIdx.x; c < pieces; c += kCastThreads) {
      float v[8];
      if (c < src_pieces) cast_load8<AT, VEC>(src, m, K, c * 8, v);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
      }
      drow[c] = cast_store8(v, s);
    }
    if (threadIdx.x == 0) rs[m] = ldexpf(1.0f, -s);
  }
}

template <int AT, bool VEC>
static void launch_cast_rows(const void* src, int64_t M, int64_t K, int64_t Kp, uint16_t* dst, float* rs,
                             hipStream_t st) {
  if (Kp <= (int64_t)kCastThreads * 8 * kCastPieces)
    launch((cast_rows_f16_kernel<AT, VEC, true>), dim3((unsigned)M), dim3(kCastThreads), 0, st, src,
                       M, K, Kp, dst, rs);
  else
    launch((cast_rows_f16_kernel<AT, VEC, false>), dim3((unsigned)M), dim3(kCastThreads), 0, st, src,
                       M, K, Kp, dst, rs);
}

template <int AT>
static void launch_cast_at(const void* src, int64_t M, int64_t K, int64_t Kp, uint16_t* dst, float* rs,
                           bool vec, hipStream_t st) {
  if (vec) launch_cast_rows<AT, true>(src, M, K, Kp, dst, rs, st);
  else launch_cast_rows<AT, false>(src, M, K, Kp, dst, rs, st);
}

hipError_t launch_cast_pad_f16(const void* src, int src_type, int64_t M, int64_t K, int64_t Kp,
                               uint16_t* dst, float* row_scale, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const bool vec = K % 8 == 0 && (uintptr_t)src % 16 == 0;
  if (src_type == QMM_F32) launch_cast_at<QMM_F32>(src, M, K, Kp, dst, row_scale, vec, st);
  else if (src_type == QMM_F16) launch_cast_at<QMM_F16>(src, M, K, Kp, dst, row_scale, vec, st);
  else launch_cast_at<QMM_BF16>(src, M, K, Kp, dst, row_scale, vec, st);
  return hipSuccess;
}

}  // namespace qmm
