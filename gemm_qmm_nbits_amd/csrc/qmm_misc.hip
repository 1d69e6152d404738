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
    const uint32_t q = code_at(d.W + n * d.row_bytes + (int64_t)b * blob, j, d.bits);
    float w;
    if (d.fmt == GEMV_CODEBOOK) {
      w = __fmul_rn(d.codebook[q], d.absmax[n * d.nblk + b]);
    } else {
      const float s = f16_to_f32(d.scales[n * d.nblk + b]);
      const float z = zero_point(d.zp, d.zp_kind, d.uniform_zp, d.bits, n, b, d.zp_row_bytes, d.nblk);
      w = dequant_affine(q, z, s);
    }
    if (d.out_type == QMM_F16) ((uint16_t*)d.out)[i] = f32_to_f16(w);
    else ((float*)d.out)[i] = w;
  }
}

hipError_t launch_dequant(const DequantArgs& d, hipStream_t st) {
  const int64_t total = d.N * d.K;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, d);
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
  hipLaunchKernelGGL(uniform_partial_kernel, dim3(kUniformPartials), dim3(256), 0, st, zp, count,
                     scratch + 2);
  hipLaunchKernelGGL(uniform_final_kernel, dim3(1), dim3(256), 0, st, zp, scratch + 2, scratch);
  return hipSuccess;
}

// ---- A cast to fp16 (prefill path; [P1] "What", commit 1: cast A once) --------
// One thread per 8 consecutive elements of a destination row (one 16-byte store).
__global__ __launch_bounds__(256) void cast_pad_f16_kernel(const void* src, int src_type, int64_t M,
                                                           int64_t K, int64_t Kp, uint16_t* dst) {
  const int64_t per_row = Kp / 8;
  const int64_t total = M * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / per_row;
    const int64_t k = (i - m * per_row) * 8;
    const int64_t base = m * K + k;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v0 = (k + 2 * e < K) ? load_elem_rt(src, src_type, base + 2 * e) : 0.0f;
      const float v1 = (k + 2 * e + 1 < K) ? load_elem_rt(src, src_type, base + 2 * e + 1) : 0.0f;
      o[e] = (uint32_t)f32_to_f16(v0) | ((uint32_t)f32_to_f16(v1) << 16);
    }
    ((uint4*)dst)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Same result for K a multiple of 8 and a 16-byte aligned source: a group of 8
// destination elements then lies wholly inside the row or wholly in the padding, and
// its source is one or two aligned 16-byte loads (vector loads, no per-element type
// switch or bounds check).  The conversion is the one above.
template <int AT>
__global__ __launch_bounds__(256) void cast_pad_f16_vec_kernel(const void* src, int64_t M, int64_t K,
                                                               int64_t Kp, uint16_t* dst) {
  const int64_t per_row = Kp / 8;
  const int64_t per_src = K / 8;
  const int64_t total = M * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / per_row;
    const int64_t c = i - m * per_row;
    uint4 out = make_uint4(0u, 0u, 0u, 0u);
    if (c < per_src) {
      const int64_t base = m * K + c * 8;
      float v[8];
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
      out.x = (uint32_t)f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16);
      out.y = (uint32_t)f32_to_f16(v[2]) | ((uint32_t)f32_to_f16(v[3]) << 16);
      out.z = (uint32_t)f32_to_f16(v[4]) | ((uint32_t)f32_to_f16(v[5]) << 16);
      out.w = (uint32_t)f32_to_f16(v[6]) | ((uint32_t)f32_to_f16(v[7]) << 16);
    }
    ((uint4*)dst)[i] = out;
  }
}

hipError_t launch_cast_pad_f16(const void* src, int src_type, int64_t M, int64_t K, int64_t Kp,
                               uint16_t* dst, hipStream_t st) {
  int64_t blocks = (M * (Kp / 8) + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (K % 8 == 0 && (uintptr_t)src % 16 == 0) {
    if (src_type == QMM_F32)
      hipLaunchKernelGGL(cast_pad_f16_vec_kernel<QMM_F32>, dim3((unsigned)blocks), dim3(256), 0, st,
                         src, M, K, Kp, dst);
    else if (src_type == QMM_F16)
      hipLaunchKernelGGL(cast_pad_f16_vec_kernel<QMM_F16>, dim3((unsigned)blocks), dim3(256), 0, st,
                         src, M, K, Kp, dst);
    else
      hipLaunchKernelGGL(cast_pad_f16_vec_kernel<QMM_BF16>, dim3((unsigned)blocks), dim3(256), 0, st,
                         src, M, K, Kp, dst);
    return hipSuccess;
  }
  hipLaunchKernelGGL(cast_pad_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, src_type, M,
                     K, Kp, dst);
  return hipSuccess;
}

}  // namespace qmm
