// Fused top-k MoE decode with u4 expert weights ([P2] hip-ep PR 1328, "Summary",
// "Why", "What": fc1 -> SwiGLU -> fc2 over the k routed experts of each token, fp
// and int8-activation ("dp4a") variants, fixed reduction order so every call
// gives the same bits).
//
// Two kernels on the caller's stream:
//   fc1: for each (token t, slot j) and row i < I, the dot products of rows i (g)
//        and I+i (u) of W1_e with x_t, plus bias, then h = fp16(g*sigmoid(g)*u)
//        stored in scratch.
//   fc2: for each token t and output row n < H, for j = 0..k-1 in order,
//        z_j = W2_e[n] . h_tj + b2_e[n] and y += w_tj * z_j; Y = fp16(y).
// Weight rows are streamed as 16-byte chunks (32 codes = one 32-value activation
// group, inside one block since block >= 32); each row is owned by LPR lanes with
// the lane->chunk map fixed by the row length, and lane partials are combined
// by a fixed xor butterfly, exactly as in the dense GEMV.
//
// Int8-activation mode: each work-group quantizes the activations it needs into
// LDS (per 32 values: amax, scale fp32(amax/127), codes rint(fp32(v * fp32(127/amax)))
// clamped to +-127), then sum(q * xq) over a chunk is exact in int32 with the
// int8 dot4 instruction (codes 0..15 are non-negative int8) and the zero point is folded as
// sum((q - zp) * xq) = sum(q * xq) - zp * sum(xq).
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// ---- shared pieces ------------------------------------------------------------

// Eight fp16 values (one 16-byte load) -> fp32.
__device__ __forceinline__ void h8_to_f32(uint4 v, float* o) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = f16_to_f32((uint16_t)(d[i] & 0xffffu));
    o[2 * i + 1] = f16_to_f32((uint16_t)(d[i] >> 16));
  }
}

// fp dot of one 16-byte chunk of u4 codes (32 codes) with 32 fp32 activations,
// unscaled: sum a[i] * q[i].  Codes are decoded two at a time through the fp8
// conversion (bytes 0..15 -> q * 2^-9), the factor 512 is applied by the caller.
__device__ __forceinline__ float dot_chunk_u4(uint4 w, const float* a) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = d[i] & 0x0f0f0f0fu;
    const uint32_t hi = (d[i] >> 4) & 0x0f0f0f0fu;
    const f32x2 l0 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
    const f32x2 l1 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    const f32x2 h0 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const f32x2 h1 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    const float* ai = a + 8 * i;
    s = fmaf(ai[0], l0.x, s);
    s = fmaf(ai[1], h0.x, s);
    s = fmaf(ai[2], l0.y, s);
    s = fmaf(ai[3], h0.y, s);
    s = fmaf(ai[4], l1.x, s);
    s = fmaf(ai[5], h1.x, s);
    s = fmaf(ai[6], l1.y, s);
    s = fmaf(ai[7], h1.y, s);
  }
  return s;
}

// int8 dot of one chunk: sum q[i] * xq[i], exact.  `xq` holds the 32 codes of the
// group permuted per 8 values as [x0 x2 x4 x6 | x1 x3 x5 x7] (two dwords).
__device__ __forceinline__ int dot_chunk_u4_i8(uint4 w, const uint32_t* xq) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = d[i] & 0x0f0f0f0fu;         // codes 0,2,4,6 of these 8
    const uint32_t hi = (d[i] >> 4) & 0x0f0f0f0fu;  // codes 1,3,5,7
    s = __builtin_amdgcn_sdot4((int)lo, (int)xq[2 * i], s, false);
    s = __builtin_amdgcn_sdot4((int)hi, (int)xq[2 * i + 1], s, false);
  }
  return s;
}

__device__ __forceinline__ float u4_zero_point(const uint8_t* zp, int64_t row, int64_t zp_row_bytes,
                                               int b) {
  if (!zp) return 8.0f;
  return (float)((zp[row * zp_row_bytes + (b >> 1)] >> ((b & 1) * 4)) & 0xfu);
}

// Symmetric int8 quantization of `n` fp32 values (n % 32 == 0) held by the whole
// work-group, into LDS: codes permuted per 8 as [0 2 4 6 | 1 3 5 7], one fp32
// scale and one int32 code sum per 32 values.  Optional natural-order copy to
// global memory (codes int8, scales fp32) for inspection.
template <typename LoadFn>
__device__ void quantize_groups_lds(LoadFn load, int n, uint32_t* q_lds, float* s_lds, int* sum_lds,
                                    int8_t* q_out, float* s_out) {
  const int groups = n / 32;
  const int lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int half = lane >> 5;        // two groups per wave pass
  const int li = lane & 31;
  for (int g0 = (threadIdx.x >> 6) * 2; g0 < groups; g0 += nwaves * 2) {
    const int g = g0 + half;
    const bool ok = g < groups;
    const float v = ok ? load(g * 32 + li) : 0.0f;
    float amax = fabsf(v);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    int q = 0;
    float s = 0.0f;
    if (amax > 0.0f) {
      const float inv = 127.0f / amax;
      const float t = __fmul_rn(v, inv);
      q = (int)rintf(t);
      q = q > 127 ? 127 : (q < -127 ? -127 : q);
      s = amax / 127.0f;
    }
    int qs = q;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) qs += __shfl_xor(qs, off, 64);
    if (ok) {
      // permuted position: within each run of 8, even indices first
      const int r = li & 7;
      const int pos = (li & ~7) + ((r & 1) ? 4 + (r >> 1) : (r >> 1));
      ((int8_t*)q_lds)[g * 32 + pos] = (int8_t)q;
      if (q_out) q_out[g * 32 + li] = (int8_t)q;
      if (li == 0) {
        s_lds[g] = s;
        sum_lds[g] = qs;
        if (s_out) s_out[g] = s;
      }
    }
  }
}

// ---- fc1 + SwiGLU ---------------------------------------------------------------

template <int INT8, int RI>
__global__ __launch_bounds__(256) void qmoe_fc1_kernel(QmoeArgs a) {
  extern __shared__ uint32_t smem[];
  const int slot = blockIdx.y;  // t * k + j
  const int t = slot / a.k;
  const int e = a.ids[slot];
  const uint16_t* x = a.X + (int64_t)t * a.H;
  const int64_t nchunks = a.fc1_chunks;  // chunks holding codes k < H
  const int64_t nblk = a.fc1_nblk;

  // int8 mode: quantize x_t into LDS (work-group (0, slot t*k) keeps a copy)
  uint32_t* xq = smem;
  float* xs = (float*)(smem + a.H / 4);
  int* xsum = (int*)(xs + a.H / 32);
  if constexpr (INT8) {
    const bool keep = blockIdx.x == 0 && (slot % a.k) == 0;
    quantize_groups_lds([&](int i) { return f16_to_f32(x[i]); }, (int)a.H, xq, xs, xsum,
                        keep ? a.xq_out + (int64_t)t * a.H : nullptr,
                        keep ? a.xs_out + (int64_t)t * (a.H / 32) : nullptr);
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int LPR = 1 << a.fc1_lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> a.fc1_lpr_log2;
  const int SUBS = 64 >> a.fc1_lpr_log2;
  const int64_t i0 = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) * (SUBS * RI) + sub;

  const uint8_t* W = a.fc1.W + (int64_t)e * 2 * a.I * a.fc1_row_bytes;
  const uint16_t* S = a.fc1.scales + (int64_t)e * 2 * a.I * nblk;
  const uint8_t* Z = a.fc1.zp ? a.fc1.zp + (int64_t)e * 2 * a.I * a.fc1_zp_row_bytes : nullptr;

  int64_t rows[2 * RI];
  bool valid[2 * RI];
#pragma unroll
  for (int r = 0; r < RI; ++r) {
    const int64_t i = i0 + (int64_t)r * SUBS;
    rows[2 * r] = i;          // g row
    rows[2 * r + 1] = i + a.I;  // u row
    valid[2 * r] = valid[2 * r + 1] = i < a.I;
  }
  float acc[2 * RI];
#pragma unroll
  for (int r = 0; r < 2 * RI; ++r) acc[r] = 0.0f;

  for (int64_t c = lp; c < nchunks; c += LPR) {
    uint4 w[2 * RI];
#pragma unroll
    for (int r = 0; r < 2 * RI; ++r)
      w[r] = valid[r] ? *(const uint4*)(W + rows[r] * a.fc1_row_bytes + c * 16) : make_uint4(0, 0, 0, 0);
    const int64_t k0 = c * 32;
    const int b = (int)(k0 / a.block);
    if constexpr (INT8) {
      const uint4 q0 = *(const uint4*)(xq + c * 8);
      const uint4 q1 = *(const uint4*)(xq + c * 8 + 4);
      const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const float sx = xs[c];
      const int sum = xsum[c];
#pragma unroll
      for (int r = 0; r < 2 * RI; ++r) {
        if (!valid[r]) continue;
        const int dotv = dot_chunk_u4_i8(w[r], qq);
        const int zp = (int)u4_zero_point(Z, rows[r], a.fc1_zp_row_bytes, b);
        const float sw = f16_to_f32(S[rows[r] * nblk + b]);
        acc[r] = fmaf(sw * sx, (float)(dotv - zp * sum), acc[r]);
      }
    } else {
      float xa[32];
      const bool full = k0 + 32 <= a.H;
      if (full) {
#pragma unroll
        for (int q = 0; q < 4; ++q) h8_to_f32(*(const uint4*)(x + k0 + 8 * q), xa + 8 * q);
      } else {
#pragma unroll
        for (int q = 0; q < 32; ++q) xa[q] = (k0 + q < a.H) ? f16_to_f32(x[k0 + q]) : 0.0f;
      }
      float sa = 0.0f;
#pragma unroll
      for (int q = 0; q < 32; ++q) sa += xa[q];
#pragma unroll
      for (int r = 0; r < 2 * RI; ++r) {
        if (!valid[r]) continue;
        const float p = dot_chunk_u4(w[r], xa);
        const float zp = u4_zero_point(Z, rows[r], a.fc1_zp_row_bytes, b);
        const float sw = f16_to_f32(S[rows[r] * nblk + b]);
        acc[r] = fmaf(sw, fmaf(-zp, sa, 512.0f * p), acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 2 * RI; ++r) acc[r] = group_sum(acc[r], LPR);
  if (lp == 0) {
#pragma unroll
    for (int r = 0; r < RI; ++r) {
      if (!valid[2 * r]) continue;
      const int64_t i = rows[2 * r];
      float g = acc[2 * r], u = acc[2 * r + 1];
      if (a.fc1.bias) {
        const uint16_t* bb = a.fc1.bias + (int64_t)e * 2 * a.I;
        g += f16_to_f32(bb[i]);
        u += f16_to_f32(bb[i + a.I]);
      }
      const float h = g / (1.0f + expf(-g)) * u;
      a.h[(int64_t)slot * a.I + i] = f32_to_f16(h);
    }
  }
}

// ---- fc2 + weighted combine -----------------------------------------------------

template <int INT8, int R>
__global__ __launch_bounds__(256) void qmoe_fc2_kernel(QmoeArgs a) {
  extern __shared__ uint32_t smem[];
  const int t = blockIdx.y;
  const int k = a.k;
  const int64_t nchunks = a.fc2_chunks;  // chunks holding codes k < I
  const int64_t nblk = a.fc2_nblk;
  const uint16_t* hT = a.h + (int64_t)t * k * a.I;  // [k][I] fp16

  uint32_t* hq = smem;                                   // [k][I] permuted codes
  float* hs = (float*)(smem + (int64_t)k * a.I / 4);     // [k][I/32]
  int* hsum = (int*)(hs + (int64_t)k * a.I / 32);        // [k][I/32]
  if constexpr (INT8) {
    const bool keep = blockIdx.x == 0;
    quantize_groups_lds([&](int i) { return f16_to_f32(hT[i]); }, (int)(k * a.I), hq, hs, hsum,
                        keep ? a.hq_out + (int64_t)t * k * a.I : nullptr,
                        keep ? a.hs_out + (int64_t)t * k * (a.I / 32) : nullptr);
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int LPR = 1 << a.fc2_lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> a.fc2_lpr_log2;
  const int SUBS = 64 >> a.fc2_lpr_log2;
  const int64_t n0 = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) * (SUBS * R) + sub;

  int64_t rows[R];
  bool valid[R];
  float y[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rows[r] = n0 + (int64_t)r * SUBS;
    valid[r] = rows[r] < a.H;
    y[r] = 0.0f;
  }

  for (int j = 0; j < k; ++j) {
    const int e = a.ids[t * k + j];
    const float rw = a.rw[t * k + j];
    const uint8_t* W = a.fc2.W + (int64_t)e * a.H * a.fc2_row_bytes;
    const uint16_t* S = a.fc2.scales + (int64_t)e * a.H * nblk;
    const uint8_t* Z = a.fc2.zp ? a.fc2.zp + (int64_t)e * a.H * a.fc2_zp_row_bytes : nullptr;
    const uint16_t* hj = hT + (int64_t)j * a.I;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    for (int64_t c = lp; c < nchunks; c += LPR) {
      uint4 w[R];
#pragma unroll
      for (int r = 0; r < R; ++r)
        w[r] = valid[r] ? *(const uint4*)(W + rows[r] * a.fc2_row_bytes + c * 16) : make_uint4(0, 0, 0, 0);
      const int64_t k0 = c * 32;
      const int b = (int)(k0 / a.block);
      if constexpr (INT8) {
        const uint32_t* qg = hq + ((int64_t)j * a.I + k0) / 4;
        const uint4 q0 = *(const uint4*)(qg);
        const uint4 q1 = *(const uint4*)(qg + 4);
        const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        const int gi = (int)((j * a.I + k0) / 32);
        const float sx = hs[gi];
        const int sum = hsum[gi];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (!valid[r]) continue;
          const int dotv = dot_chunk_u4_i8(w[r], qq);
          const int zp = (int)u4_zero_point(Z, rows[r], a.fc2_zp_row_bytes, b);
          const float sw = f16_to_f32(S[rows[r] * nblk + b]);
          acc[r] = fmaf(sw * sx, (float)(dotv - zp * sum), acc[r]);
        }
      } else {
        float xa[32];
        const bool full = k0 + 32 <= a.I;
        if (full) {
#pragma unroll
          for (int q = 0; q < 4; ++q) h8_to_f32(*(const uint4*)(hj + k0 + 8 * q), xa + 8 * q);
        } else {
#pragma unroll
          for (int q = 0; q < 32; ++q) xa[q] = (k0 + q < a.I) ? f16_to_f32(hj[k0 + q]) : 0.0f;
        }
        float sa = 0.0f;
#pragma unroll
        for (int q = 0; q < 32; ++q) sa += xa[q];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (!valid[r]) continue;
          const float p = dot_chunk_u4(w[r], xa);
          const float zp = u4_zero_point(Z, rows[r], a.fc2_zp_row_bytes, b);
          const float sw = f16_to_f32(S[rows[r] * nblk + b]);
          acc[r] = fmaf(sw, fmaf(-zp, sa, 512.0f * p), acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float z = group_sum(acc[r], LPR) +
                      ((a.fc2.bias && valid[r]) ? f16_to_f32(a.fc2.bias[(int64_t)e * a.H + rows[r]]) : 0.0f);
      y[r] = fmaf(rw, z, y[r]);
    }
  }
  if (lp == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (valid[r]) a.Y[(int64_t)t * a.H + rows[r]] = f32_to_f16(y[r]);
  }
}

// ---- launch ---------------------------------------------------------------------

size_t qmoe_fc1_lds_bytes(const QmoeArgs& a) {
  return a.mode == QMOE_INT8_ACT ? (size_t)a.H + (size_t)(a.H / 32) * 8 : 0;
}
size_t qmoe_fc2_lds_bytes(const QmoeArgs& a) {
  return a.mode == QMOE_INT8_ACT ? (size_t)(a.k * a.I) + (size_t)(a.k * a.I / 32) * 8 : 0;
}

hipError_t launch_qmoe_fc1(const QmoeArgs& a, int rows_per_lane, hipStream_t st) {
  const int subs = 64 >> a.fc1_lpr_log2;
  const int64_t rows_per_wg = 4LL * subs * rows_per_lane;
  const dim3 grid((unsigned)((a.I + rows_per_wg - 1) / rows_per_wg), (unsigned)(a.T * a.k));
  const size_t lds = qmoe_fc1_lds_bytes(a);
  if (a.mode == QMOE_INT8_ACT) {
    if (rows_per_lane == 1) hipLaunchKernelGGL((qmoe_fc1_kernel<1, 1>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((qmoe_fc1_kernel<1, 2>), grid, dim3(256), lds, st, a);
  } else {
    if (rows_per_lane == 1) hipLaunchKernelGGL((qmoe_fc1_kernel<0, 1>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((qmoe_fc1_kernel<0, 2>), grid, dim3(256), 0, st, a);
  }
  return hipSuccess;
}

hipError_t launch_qmoe_fc2(const QmoeArgs& a, int rows_per_lane, hipStream_t st) {
  const int subs = 64 >> a.fc2_lpr_log2;
  const int64_t rows_per_wg = 4LL * subs * rows_per_lane;
  const dim3 grid((unsigned)((a.H + rows_per_wg - 1) / rows_per_wg), (unsigned)a.T);
  const size_t lds = qmoe_fc2_lds_bytes(a);
  if (a.mode == QMOE_INT8_ACT) {
    if (rows_per_lane == 1) hipLaunchKernelGGL((qmoe_fc2_kernel<1, 1>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((qmoe_fc2_kernel<1, 2>), grid, dim3(256), lds, st, a);
  } else {
    if (rows_per_lane == 1) hipLaunchKernelGGL((qmoe_fc2_kernel<0, 1>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((qmoe_fc2_kernel<0, 2>), grid, dim3(256), 0, st, a);
  }
  return hipSuccess;
}

}  // namespace qmm
