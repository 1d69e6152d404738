// Device-side helpers shared by the gfx950 kernels of the qmm library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---- scalar conversions (all round to nearest even) -------------------------

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 v = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  uint16_t h;
  __builtin_memcpy(&h, &v, 2);
  return h;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int T>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (T == QMM_F32) return ((const float*)p)[i];
  else if constexpr (T == QMM_F16) return f16_to_f32(((const uint16_t*)p)[i]);
  else return bf16_to_f32(((const uint16_t*)p)[i]);
}

__device__ __forceinline__ float load_elem_rt(const void* p, int t, int64_t i) {
  if (t == QMM_F32) return ((const float*)p)[i];
  if (t == QMM_F16) return f16_to_f32(((const uint16_t*)p)[i]);
  return bf16_to_f32(((const uint16_t*)p)[i]);
}

__device__ __forceinline__ void store_elem_rt(void* p, int t, int64_t i, float v) {
  if (t == QMM_F32) ((float*)p)[i] = v;
  else if (t == QMM_F16) ((uint16_t*)p)[i] = f32_to_f16(v);
  else ((uint16_t*)p)[i] = f32_to_bf16(v);
}

// ---- code extraction -------------------------------------------------------

// Code of element j (0-based) of a packed block: bits = 2, 3, 4 give the unsigned field
// at bit j * bits of the block's little-endian bit stream (a 3-bit field may continue
// into the next byte, which is read only then); bits = 8 gives the signed byte.
__device__ __forceinline__ int32_t code_at(const uint8_t* blk, int j, int bits) {
  if (bits == 8) return (int32_t)(int8_t)blk[j];
  const int bit = j * bits;
  uint32_t v = blk[bit >> 3];
  if ((bit & 7) + bits > 8) v |= (uint32_t)blk[(bit >> 3) + 1] << 8;
  return (int32_t)((v >> (bit & 7)) & ((1u << bits) - 1u));
}

// Zero point when none is given: the middle code of unsigned codes, 0 for signed int8.
__host__ __device__ __forceinline__ float default_zero_point(int bits) {
  return bits == 8 ? 0.0f : (float)(1 << (bits - 1));
}

// Zero point of (row n, block b) as fp32 for each zero-point kind (packed zero points use
// the weights' field layout: block b is field b of the row's bit stream).
__device__ __forceinline__ float zero_point(const void* zp, int zp_kind, float uniform_zp,
                                            int bits, int64_t n, int b, int64_t zp_row_bytes,
                                            int64_t nblk) {
  switch (zp_kind) {
    case QMM_ZP_PACKED:
      return (float)code_at((const uint8_t*)zp + n * zp_row_bytes, b, bits);
    case QMM_ZP_F16:
      return f16_to_f32(((const uint16_t*)zp)[n * nblk + b]);
    case QMM_ZP_UNIFORM:
      return uniform_zp;
    default:
      return default_zero_point(bits);
  }
}

// Bit-exact affine dequant: fp32(fp32(q - zp) * s), two separate roundings.
__device__ __forceinline__ float dequant_affine(int32_t q, float zp, float s) {
  float d = __fsub_rn((float)q, zp);
  return __fmul_rn(d, s);
}

// The fp32 value as a register a following conversion reads: keeps the compiler from
// merging the operation that produced it with a conversion to a 16-bit type (a mixed-
// precision operation would round the exact result once, not the fp32 value).
__device__ __forceinline__ float materialize(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ---- wave-level helpers ------------------------------------------------------

// xor-swizzle inside groups of 32 lanes (ds_swizzle bit mode: and 0x1f, xor k)
template <int K>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (K << 10)));
}

// Raw buffer descriptor (32-bit data format) over `bytes` bytes at p: loads past the
// range return 0 and fetch nothing.
constexpr uint32_t kBufferWord3 = 0x00020000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kBufferWord3);
}

// Lane exchange inside rows of 16 lanes through DPP (no LDS traffic): xor 1 and
// xor 2 inside quads, then the mirror of each half row (lane i <-> 7 - i) and of the
// row (lane i <-> 15 - i).  Applied in that order with a commutative combine, every
// lane of an aligned group of 4, 8 or 16 lanes ends with the same group result.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Butterfly sum over groups of `width` consecutive lanes (power of two <= 64).
// Every lane of the group ends with the same, order-fixed result: at each step a
// lane adds its partner's value (a + b == b + a bitwise, so partners agree).
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width > 1) v += swz_xor<1>(v);
  if (width > 2) v += swz_xor<2>(v);
  if (width > 4) v += swz_xor<4>(v);
  if (width > 8) v += swz_xor<8>(v);
  if (width > 16) v += swz_xor<16>(v);
  if (width > 32) v += __shfl_xor(v, 32, 64);
  return v;
}

}  // namespace qmm
