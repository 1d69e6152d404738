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
#include "qmm_qmoe.h"

#include <map>
#include <mutex>
#include <type_traits>

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

// Staged fp activations are fp16 pairs: each 8 values x0..x7 are held as the four
// dwords (x0,x2) (x4,x6) (x1,x3) (x5,x7), the order in which the code decoding below
// yields the codes (low nibbles give codes 0,2,4,6, high nibbles 1,3,5,7).
__device__ __forceinline__ uint4 h8_pairs(uint4 v) {
  const uint32_t p02 = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
  const uint32_t p46 = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
  const uint32_t p13 = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
  const uint32_t p57 = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
  return make_uint4(p02, p46, p13, p57);
}

// fp dot of one 16-byte chunk of u4 codes (32 codes) with its 32 staged activations
// (16 dwords of fp16 pairs), unscaled: sum q[i] * a[i].  Each byte holding a code is
// read as an fp8 E4M3 value (codes 0..15 are q * 2^-9) and converted to fp16 with the
// scale 2^9, which gives q exactly; the pairs go through the fp16 dot into the fp32
// sum (products of fp16 values are exact in fp32), in a fixed order.
typedef _Float16 moe_h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot_chunk_u4(uint4 w, const uint32_t* a) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = d[i] & 0x0f0f0f0fu;         // codes 0,2,4,6 of these 8
    const uint32_t hi = (d[i] >> 4) & 0x0f0f0f0fu;  // codes 1,3,5,7
    const moe_h2 q02 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);
    const moe_h2 q46 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);
    const moe_h2 q13 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);
    const moe_h2 q57 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);
    const uint32_t* ai = a + 4 * i;
    s = __builtin_amdgcn_fdot2(q02, __builtin_bit_cast(moe_h2, ai[0]), s, false);
    s = __builtin_amdgcn_fdot2(q46, __builtin_bit_cast(moe_h2, ai[1]), s, false);
    s = __builtin_amdgcn_fdot2(q13, __builtin_bit_cast(moe_h2, ai[2]), s, false);
    s = __builtin_amdgcn_fdot2(q57, __builtin_bit_cast(moe_h2, ai[3]), s, false);
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

// ---- staged activations ------------------------------------------------------------
//
// fp mode: the activation vector in LDS as fp16 pairs, 16 dwords per 32-value chunk
// (h8_pairs order, zero past the end) at a stride of kPairStride dwords, and the
// fixed-order fp32 sum of each chunk (for the zero-point fold).
// int8 mode: codes permuted per 8 as [0 2 4 6 | 1 3 5 7], one fp32 scale and one
// int32 code sum per 32 values.

// Staged chunks lie kPairStride dwords apart: the pad dword puts the chunks that
// consecutive lanes read in different LDS banks (at 16 dwords every fourth lane would
// share a bank).
constexpr int kPairStride = 17;
// cache-policy bit sc1 of a load: device scope (misses the L2, so it sees what other
// work-groups of the same launch wrote through theirs)
constexpr int kDeviceCoherent = 16;
__device__ __forceinline__ void store_pairs(uint32_t* p, uint4 v) {
  p[0] = v.x;
  p[1] = v.y;
  p[2] = v.z;
  p[3] = v.w;
}
__device__ __forceinline__ uint4 load_pairs(const uint32_t* p) { return make_uint4(p[0], p[1], p[2], p[3]); }

// Staging of `rows` vectors of n fp16 values each (row stride n, 16-byte aligned
// rows): xh[r][nch][kPairStride] (fp16 pairs, zero past n) and the chunk sums sa[r][nch], in
// one pass: each thread takes 8 values, and the 4 threads of a chunk (one quad of
// lanes) combine their fp32 sums of 8 through DPP in a fixed order.
__device__ __forceinline__ void stage_h16(const uint16_t* src, int rows, int n, int nch, uint32_t* xh, float* sa) {
  const int per_row = nch * 4;  // pieces of 8 values
  const int total = rows * per_row;
  for (int p = threadIdx.x; p < total; p += blockDim.x) {  // quads are all in or all out
    const int r = p / per_row;
    const int pp = p - r * per_row;
    const int k0 = 8 * pp;
    const uint16_t* row = src + (int64_t)r * n;
    uint4 u;
    if (k0 + 8 <= n) {
      u = *(const uint4*)(row + k0);
    } else {
      uint16_t h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = k0 + q < n ? row[k0 + q] : (uint16_t)0;
      u = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16), h[4] | ((uint32_t)h[5] << 16),
                     h[6] | ((uint32_t)h[7] << 16));
    }
    float v[8];
    h8_to_f32(u, v);
    store_pairs(xh + ((int64_t)r * nch + (k0 >> 5)) * kPairStride + ((k0 & 31) >> 1), h8_pairs(u));
    float s8 = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    s8 += dpp_f<kDppXor1>(s8);
    s8 += dpp_f<kDppXor2>(s8);
    if ((pp & 3) == 0) sa[r * nch + (pp >> 2)] = s8;
  }
  __syncthreads();
}

// The same staging (same values and sums) with the loads of the first batch (NB
// pieces per thread) issued before `issued` runs: a caller that starts its weight
// loads there has them travel while the activations are converted, and waiting for
// the activations, which were issued first, does not wait for them.  Every batch has
// all its loads in flight at once.  AUX: the loads' cache-policy bits (device-coherent
// loads for values other work-groups of the same launch wrote).
template <int AUX = 0, typename Issued>
__device__ __forceinline__ void stage_h16_first(const uint16_t* src, int rows, int n, int nch, uint32_t* xh,
                                                float* sa, Issued&& issued) {
  constexpr int NB = 4;
  const int per_row = nch * 4;  // pieces of 8 values
  const int total = rows * per_row;
  const int wave_base = __builtin_amdgcn_readfirstlane((int)(threadIdx.x & ~63u));
  // n % 8 == 0 (checked at the entry point): a piece is wholly inside the row or
  // wholly past it.  Every lane issues its loads unconditionally: a piece past the row
  // or past the batch loads from beyond the descriptor's range, which returns zero and
  // moves no data (a load inside a branch would make the compiler wait for it at the
  // branch's end, before the caller's loads are issued).
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)rows * (uint32_t)n * 2u);
  auto load = [&](int p, uint4& u) {
    const bool okp = p < total;
    const int pc = okp ? p : 0;
    const int r = pc / per_row;
    const int k0 = 8 * (pc - r * per_row);
    const uint32_t off = okp && k0 < n ? ((uint32_t)r * (uint32_t)n + (uint32_t)k0) * 2u : 0x80000000u;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, AUX);
    u = make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto convert = [&](int p, const uint4& u) {
    const bool okp = p < total;
    const int pc = okp ? p : 0;
    const int r = pc / per_row;
    const int pp = pc - r * per_row;
    const int k0 = 8 * pp;
    if (okp) store_pairs(xh + ((int64_t)r * nch + (k0 >> 5)) * kPairStride + ((k0 & 31) >> 1), h8_pairs(u));
    float v[8];
    h8_to_f32(u, v);
    float s8 = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    s8 += dpp_f<kDppXor1>(s8);
    s8 += dpp_f<kDppXor2>(s8);
    if (okp && (pp & 3) == 0) sa[r * nch + (pp >> 2)] = s8;
  };
  auto batch = [&](int base, auto first) {
    uint4 vb[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) load(base + j * (int)blockDim.x + (int)threadIdx.x, vb[j]);
    if constexpr (decltype(first)::value) {
      __builtin_amdgcn_sched_barrier(0);  // keep the caller's loads behind these
      issued();
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (base + j * (int)blockDim.x + wave_base < total) convert(base + j * (int)blockDim.x + (int)threadIdx.x, vb[j]);
  };
  batch(0, std::true_type{});
  for (int base = NB * (int)blockDim.x; base < total; base += NB * (int)blockDim.x) batch(base, std::false_type{});
  __syncthreads();
}

// int8 staging of the n fp16 values at src (n % 32 == 0, 16-byte aligned; rows back to
// back, each a multiple of 32 values): 16-byte loads of 8 values per lane, so the 4
// lanes of a quad hold one 32-value group, NB per thread in flight at once; the group
// is quantized as the oracle's quantizer does it (amax over the 32 values, codes
// rint(v * fp32(127/amax)) clamped to +-127, scale fp32(amax/127); all zero when amax
// is 0), the codes go to LDS permuted per 8 as [0 2 4 6 | 1 3 5 7], with the scale and
// the code sum per group.  q_out / s_out (may be null): the codes in natural order and
// the scales, in memory.  The first batch's loads are issued before `issued` runs (as
// in stage_h16_first).  AUX: the loads' cache-policy bits.
template <int AUX, typename Issued>
__device__ __forceinline__ void stage_i8_first(const uint16_t* src, int n, uint32_t* q_lds, float* s_lds,
                                               int* sum_lds, int8_t* q_out, float* s_out, Issued&& issued) {
  constexpr int NB = 4;
  const int total = n / 8;  // pieces of 8 values, a multiple of 4: quads are all in or all out
  const int wave_base = __builtin_amdgcn_readfirstlane((int)(threadIdx.x & ~63u));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)n * 2u);
  auto load = [&](int p, uint4& u) {
    const uint32_t off = p < total ? (uint32_t)p * 16u : 0x80000000u;  // past the range: 0, no data
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, AUX);
    u = make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto pack = [](int a0, int a1, int a2, int a3) {
    return (uint32_t)(a0 & 0xff) | ((uint32_t)(a1 & 0xff) << 8) | ((uint32_t)(a2 & 0xff) << 16) |
           ((uint32_t)(a3 & 0xff) << 24);
  };
  auto convert = [&](int p, const uint4& u) {
    float v[8];
    h8_to_f32(u, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
    int q[8];
    float sc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = 0;
    if (amax > 0.0f) {
      const float inv = 127.0f / amax;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = (int)rintf(__fmul_rn(v[i], inv));
        q[i] = c > 127 ? 127 : (c < -127 ? -127 : c);
      }
      sc = amax / 127.0f;
    }
    int sum = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
    sum += __float_as_int(dpp_f<kDppXor1>(__int_as_float(sum)));
    sum += __float_as_int(dpp_f<kDppXor2>(__int_as_float(sum)));
    if (p < total) {
      const int g = p >> 2, m = p & 3;
      q_lds[g * 8 + 2 * m] = pack(q[0], q[2], q[4], q[6]);
      q_lds[g * 8 + 2 * m + 1] = pack(q[1], q[3], q[5], q[7]);
      if (m == 0) {
        s_lds[g] = sc;
        sum_lds[g] = sum;
      }
      if (q_out) {
        *(uint2*)(q_out + (int64_t)p * 8) = make_uint2(pack(q[0], q[1], q[2], q[3]), pack(q[4], q[5], q[6], q[7]));
        if (m == 0) s_out[g] = sc;
      }
    }
  };
  auto batch = [&](int base, auto first) {
    uint4 vb[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) load(base + j * (int)blockDim.x + (int)threadIdx.x, vb[j]);
    if constexpr (decltype(first)::value) {
      __builtin_amdgcn_sched_barrier(0);  // keep the caller's loads behind these
      issued();
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (base + j * (int)blockDim.x + wave_base < total) convert(base + j * (int)blockDim.x + (int)threadIdx.x, vb[j]);
  };
  batch(0, std::true_type{});
  for (int base = NB * (int)blockDim.x; base < total; base += NB * (int)blockDim.x) batch(base, std::false_type{});
  __syncthreads();
}

// int8 staging from codes already quantized (natural order) and their scales.
__device__ __forceinline__ void stage_i8(const int8_t* q, const float* sc, int n, uint32_t* q_lds,
                                         float* s_lds, int* sum_lds) {
  const int groups = n / 32;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int r = i & 7;
    const int pos = (i & ~7) + ((r & 1) ? 4 + (r >> 1) : (r >> 1));
    ((int8_t*)q_lds)[pos] = q[i];
  }
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    int v = 0;
    for (int i = 0; i < 32; ++i) v += q[g * 32 + i];
    s_lds[g] = sc[g];
    sum_lds[g] = v;
  }
  __syncthreads();
}

// Raw loads of one item (one 16-byte chunk of NR weight rows) of one lane.
template <int NR>
struct MoeItem {
  uint4 w[NR];
  _Float16 s[NR];
  uint32_t z[NR];  // packed zero-point byte (unshifted)
};

constexpr int kMoeThreads = 256;
// LDS dwords per staged 32-value chunk in fp mode: kPairStride of fp16 pairs (one pad)
// and the chunk sum
constexpr int kStagedWords = kPairStride + 1;
// slots (T * k) up to which the fc1 form that reads each expert once per call applies
constexpr int kMoeSortSlots = 64;
constexpr int kMoeStreamThreads = 512;  // persistent forms

// Expert ids outside [0, E) (a caller error) are clamped into it: never a fault.
__device__ __forceinline__ int clamp_expert(int e, int64_t E) {
  return e < 0 ? 0 : (e >= (int)E ? (int)E - 1 : e);
}
// items per lane whose loads are in flight (ring of register sets): fc1 items carry
// 2 * RI rows (register-heavy), fc2 items one row per R
constexpr int kFc1Depth = 2;
constexpr int kFc2Depth = 4;

// ---- fc1 + SwiGLU ---------------------------------------------------------------

// Work-group (row tile, slot t*k + j): rows i of the tile, for each the g row i and the
// u row I + i of W1_e; each lane walks its chunks of those 2*RI rows with the loads of
// the next chunk in flight.
template <int INT8, int RI>
__global__ __launch_bounds__(kMoeThreads) void qmoe_fc1_kernel(QmoeArgs a) {
  constexpr int NR = 2 * RI;
  extern __shared__ uint32_t smem[];
  const int slot = blockIdx.y;  // t * k + j
  const int t = slot / a.k;
  const int e = clamp_expert(a.ids[slot], a.E);
  const uint16_t* x = a.X + (int64_t)t * a.H;
  const int nch = (int)a.fc1_chunks;  // chunks holding codes k < H
  const int nblk = (int)a.fc1_nblk;

  uint32_t* xh = smem;               // fp mode
  float* sa = (float*)(xh + nch * kPairStride);
  uint32_t* xq = smem;               // int8 mode
  float* xs = (float*)(smem + a.H / 4);
  int* xsum = (int*)(xs + a.H / 32);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr_log2 = a.fc1_lpr_log2;
  const int LPR = 1 << lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> lpr_log2;
  const int SUBS = 64 >> lpr_log2;
  const int I = (int)a.I;
  const int i0 = ((int)blockIdx.x * (kMoeThreads >> 6) + wave) * (SUBS * RI) + sub;

  const uint8_t* W = a.fc1.W + (int64_t)e * 2 * a.I * a.fc1_row_bytes;
  const _Float16* S = (const _Float16*)a.fc1.scales + (int64_t)e * 2 * a.I * nblk;
  const uint8_t* Z = a.fc1.zp ? a.fc1.zp + (int64_t)e * 2 * a.I * a.fc1_zp_row_bytes : nullptr;

  int rowc[NR];  // rows clamped into the expert (loads always valid)
  bool valid[NR];
#pragma unroll
  for (int r = 0; r < RI; ++r) {
    const int i = i0 + r * SUBS;
    valid[2 * r] = valid[2 * r + 1] = i < I;
    rowc[2 * r] = i < I ? i : 0;
    rowc[2 * r + 1] = (i < I ? i : 0) + I;
  }
  const int iters = (nch + LPR - 1) >> lpr_log2;
  const int blk_shift = __builtin_ctz((unsigned)a.block) - 5;  // chunks per block = block / 32

  int fit = 0;
  auto fetch = [&](MoeItem<NR>& b) {
    int c = fit * LPR + lp;
    c = c < nch ? c : nch - 1;
    const int blk = c >> blk_shift;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      b.w[r] = *(const uint4*)(W + (int64_t)rowc[r] * a.fc1_row_bytes + c * 16);
      b.s[r] = S[(int64_t)rowc[r] * nblk + blk];
      if (Z) b.z[r] = Z[(int64_t)rowc[r] * a.fc1_zp_row_bytes + (blk >> 1)];
      else b.z[r] = 0x88u;
    }
    ++fit;
  };

  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
  int cit = 0;
  auto step = [&](const MoeItem<NR>& cb, MoeItem<NR>& nxt) {
    fetch(nxt);
    const int c = cit * LPR + lp;
    const bool cv = c < nch;
    const int cc = cv ? c : nch - 1;
    const int blk = cc >> blk_shift;
    if constexpr (INT8) {
      const uint4 q0 = *(const uint4*)(xq + cc * 8);
      const uint4 q1 = *(const uint4*)(xq + cc * 8 + 4);
      const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const float sx = xs[cc];
      const int sum = xsum[cc];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int dotv = dot_chunk_u4_i8(cb.w[r], qq);
        const int zp = (int)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
        const float nv = fmaf((float)cb.s[r] * sx, (float)(dotv - zp * sum), acc[r]);
        acc[r] = cv ? nv : acc[r];
      }
    } else {
      uint32_t xa[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = load_pairs(xh + cc * kPairStride + 4 * q);
        xa[4 * q] = v.x; xa[4 * q + 1] = v.y; xa[4 * q + 2] = v.z; xa[4 * q + 3] = v.w;
      }
      const float sac = sa[cc];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float pr = dot_chunk_u4(cb.w[r], xa);
        const float zp = (float)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
        const float nv = fmaf((float)cb.s[r], fmaf(-zp, sac, pr), acc[r]);
        acc[r] = cv ? nv : acc[r];
      }
    }
    ++cit;
  };
  // the first loads go out before the activations are staged
  MoeItem<NR> buf[kFc1Depth];
#pragma unroll
  for (int i = 0; i < kFc1Depth - 1; ++i) fetch(buf[i]);
  if constexpr (INT8) {
    const bool keep = blockIdx.x == 0 && (slot % a.k) == 0;
    stage_i8_first<0>(x, (int)a.H, xq, xs, xsum, keep ? a.xq_out + (int64_t)t * a.H : nullptr,
                      keep ? a.xs_out + (int64_t)t * (a.H / 32) : nullptr, [] {});
  } else {
    stage_h16(x, 1, (int)a.H, nch, xh, sa);
  }
  for (int base = 0; base < iters; base += kFc1Depth) {
#pragma unroll
    for (int i = 0; i < kFc1Depth; ++i) step(buf[i], buf[(i + kFc1Depth - 1) % kFc1Depth]);
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = group_sum(acc[r], LPR);
  if (lp == 0) {
#pragma unroll
    for (int r = 0; r < RI; ++r) {
      if (!valid[2 * r]) continue;
      const int i = i0 + r * SUBS;
      float g = acc[2 * r], u = acc[2 * r + 1];
      if (a.fc1.bias) {
        const uint16_t* bb = a.fc1.bias + (int64_t)e * 2 * a.I;
        g += f16_to_f32(bb[i]);
        u += f16_to_f32(bb[i + a.I]);
      }
      const float hv = g / (1.0f + expf(-g)) * u;
      a.h[(int64_t)slot * a.I + i] = f32_to_f16(hv);
    }
  }
}

// ---- int8 mode: quantization of h once per call ------------------------------------

// One half-wave per 32-value group of h [T*k][I]: codes (natural order) and scale
// into the scratch that fc2 stages from.
__global__ __launch_bounds__(256) void qmoe_quant_h_kernel(const uint16_t* h, int64_t groups, int8_t* q_out,
                                                           float* s_out) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 31;
  const int64_t g = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const bool ok = g < groups;
  const float v = ok ? f16_to_f32(h[g * 32 + li]) : 0.0f;
  float amax = fabsf(v);
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  int q = 0;
  float sc = 0.0f;
  if (amax > 0.0f) {
    const float inv = 127.0f / amax;
    q = (int)rintf(__fmul_rn(v, inv));
    q = q > 127 ? 127 : (q < -127 ? -127 : q);
    sc = amax / 127.0f;
  }
  if (ok) {
    q_out[g * 32 + li] = (int8_t)q;
    if (li == 0) s_out[g] = sc;
  }
}

// ---- fc2 + weighted combine -----------------------------------------------------

// Work-group (row tile, token t): output rows n of the tile; each lane walks the
// chunks of row n of W2_e for the k slots of the token in slot order, with the loads
// of the next item in flight across slot boundaries; at the end of slot j the lane
// partials are combined (fixed butterfly) and y += w_j * (z_j + b2).
template <int INT8, int R>
__global__ __launch_bounds__(kMoeThreads) void qmoe_fc2_kernel(QmoeArgs a) {
  extern __shared__ uint32_t smem[];
  const int t = blockIdx.y;
  const int k = a.k;
  const int nch = (int)a.fc2_chunks;  // chunks holding codes k < I
  const int nblk = (int)a.fc2_nblk;
  const int I = (int)a.I;
  const uint16_t* hT = a.h + (int64_t)t * k * a.I;  // [k][I] fp16

  uint32_t* hh = smem;                              // fp: [k][nch][kPairStride] fp16 pairs
  float* sa = (float*)(hh + (int64_t)k * nch * kPairStride);  // fp: [k][nch]
  uint32_t* hq = smem;                              // int8: [k][I] permuted codes
  float* hs = (float*)(smem + (int64_t)k * a.I / 4);
  int* hsum = (int*)(hs + (int64_t)k * a.I / 32);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr_log2 = a.fc2_lpr_log2;
  const int LPR = 1 << lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> lpr_log2;
  const int SUBS = 64 >> lpr_log2;
  const int H = (int)a.H;
  const int n0 = ((int)blockIdx.x * (kMoeThreads >> 6) + wave) * (SUBS * R) + sub;

  int rowc[R];
  bool valid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = n0 + r * SUBS;
    valid[r] = n < H;
    rowc[r] = n < H ? n : 0;
  }
  const int iters = (nch + LPR - 1) >> lpr_log2;
  const int total = k * iters;
  const int blk_shift = __builtin_ctz((unsigned)a.block) - 5;

  // fetch cursor (slot fj, item fit)
  int fj = 0, fit = 0;
  auto fetch = [&](MoeItem<R>& b) {
    const int jj = fj < k ? fj : k - 1;
    const int e = clamp_expert(a.ids[t * k + jj], a.E);
    const uint8_t* W = a.fc2.W + (int64_t)e * a.H * a.fc2_row_bytes;
    const _Float16* S = (const _Float16*)a.fc2.scales + (int64_t)e * a.H * nblk;
    int c = fit * LPR + lp;
    c = c < nch ? c : nch - 1;
    const int blk = c >> blk_shift;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      b.w[r] = *(const uint4*)(W + (int64_t)rowc[r] * a.fc2_row_bytes + c * 16);
      b.s[r] = S[(int64_t)rowc[r] * nblk + blk];
      if (a.fc2.zp)
        b.z[r] = a.fc2.zp[((int64_t)e * a.H + rowc[r]) * a.fc2_zp_row_bytes + (blk >> 1)];
      else
        b.z[r] = 0x88u;
    }
    if (++fit == iters) {
      fit = 0;
      ++fj;
    }
  };

  float acc[R], y[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = y[r] = 0.0f;
  int cj = 0, cit = 0;
  auto step = [&](const MoeItem<R>& cb, MoeItem<R>& nxt, bool live) {
    fetch(nxt);
    const int c = cit * LPR + lp;
    const bool cv = live && c < nch;
    const int cc = c < nch ? c : nch - 1;
    const int jj = cj < k ? cj : k - 1;
    const int blk = cc >> blk_shift;
    if constexpr (INT8) {
      const uint32_t* qg = hq + (jj * I + cc * 32) / 4;
      const uint4 q0 = *(const uint4*)(qg);
      const uint4 q1 = *(const uint4*)(qg + 4);
      const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const int gi = (jj * I + cc * 32) / 32;
      const float sx = hs[gi];
      const int sum = hsum[gi];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int dotv = dot_chunk_u4_i8(cb.w[r], qq);
        const int zp = (int)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
        const float nv = fmaf((float)cb.s[r] * sx, (float)(dotv - zp * sum), acc[r]);
        acc[r] = cv ? nv : acc[r];
      }
    } else {
      const uint32_t* xp = hh + ((int64_t)jj * nch + cc) * kPairStride;
      uint32_t xa[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = load_pairs(xp + 4 * q);
        xa[4 * q] = v.x; xa[4 * q + 1] = v.y; xa[4 * q + 2] = v.z; xa[4 * q + 3] = v.w;
      }
      const float sac = sa[jj * nch + cc];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pr = dot_chunk_u4(cb.w[r], xa);
        const float zp = (float)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
        const float nv = fmaf((float)cb.s[r], fmaf(-zp, sac, pr), acc[r]);
        acc[r] = cv ? nv : acc[r];
      }
    }
    if (live && cit == iters - 1) {
      // slot cj complete: z = butterfly(acc) + b2, y += w * z (slot order)
      const int e = clamp_expert(a.ids[t * k + cj], a.E);
      const float rw = a.rw[t * k + cj];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float z = group_sum(acc[r], LPR) +
                        ((a.fc2.bias && valid[r]) ? f16_to_f32(a.fc2.bias[(int64_t)e * a.H + rowc[r]]) : 0.0f);
        y[r] = fmaf(rw, z, y[r]);
        acc[r] = 0.0f;
      }
    }
    if (++cit == iters) {
      cit = 0;
      ++cj;
    }
  };
  // the first loads go out before the activations are staged
  MoeItem<R> buf[kFc2Depth];
#pragma unroll
  for (int i = 0; i < kFc2Depth - 1; ++i) fetch(buf[i]);
  if constexpr (INT8) {
    stage_i8(a.hq_out + (int64_t)t * k * a.I, a.hs_out + (int64_t)t * k * (a.I / 32), k * I, hq, hs, hsum);
  } else {
    stage_h16(hT, k, I, nch, hh, sa);
  }
  for (int base = 0; base < total; base += kFc2Depth) {
#pragma unroll
    for (int i = 0; i < kFc2Depth; ++i)
      step(buf[i], buf[(i + kFc2Depth - 1) % kFc2Depth], base + i < total);
  }
  if (lp == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (valid[r]) a.Y[(int64_t)t * a.H + n0 + r * SUBS] = f32_to_f16(y[r]);
  }
}

// ---- persistent forms (fp mode) ------------------------------------------------------
//
// One work-group per resident slot.  The activations of every token (fc1: x; fc2: the
// k rows of h of every token) are staged once per work-group, and the row groups (the
// rows one wave works on at once, all of one slot, so of one expert) are dealt out
// evenly: work-group b owns the contiguous groups [g_begin, g_end), wave w of it takes
// groups g_begin + w, g_begin + w + waves, ...  A wave's weight loads run through one
// register ring across its groups (and, in fc2, across the k slots of a group).  The
// per-row arithmetic and its order are those of the kernels above, so both forms give
// the same bits.  Row partial sums stay in LDS; bias, SwiGLU and the router-weighted
// combine run at the write-out after the loop, so no load or store other than the
// weight stream sits in the loop.  Expert ids are read with scalar loads (one per
// group or slot) and clamped into [0, E).

// COH: h is written with device-coherent stores (read by other work-groups of the
// same launch in the single-launch form).  `issued` runs once the activations' loads
// and the first weight loads are out (the single-launch form issues its fc2 weight
// copies there).
template <int RI, int ZK, bool COH, bool INT8, typename Issued>
__device__ __forceinline__ void fc1_stream_body(const QmoeArgs& a, int bid, int nb, uint32_t* smem,
                                                Issued&& issued) {
  constexpr int NR = 2 * RI;
  constexpr int NW = kMoeStreamThreads / 64;
  constexpr int D = RI == 1 ? 4 : 3;  // a wave's few items all in flight
  const int T = (int)a.T;
  const int k = a.k;
  const int I = (int)a.I;
  const int nch = (int)a.fc1_chunks;
  const int nblk = (int)a.fc1_nblk;
  const int H = (int)a.H;
  uint32_t* xh = smem;                         // fp: [T][nch][kPairStride] fp16 pairs
  float* sa = (float*)(xh + (size_t)T * nch * kPairStride);  // fp: [T][nch]
  uint32_t* xq = smem;                         // int8: [T][H / 4] permuted codes
  float* xs = (float*)(smem + (size_t)T * H / 4);  // int8: [T][H / 32] scales
  int* xsum = (int*)(xs + (size_t)T * H / 32);     // int8: [T][H / 32] code sums
  float* outs = INT8 ? (float*)(xsum + (size_t)T * H / 32) : sa + (size_t)T * nch;  // [local rows][2]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lpr_log2 = a.fc1_lpr_log2;
  const int LPR = 1 << lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> lpr_log2;
  const int SUBS = 64 >> lpr_log2;
  const int rpg = SUBS * RI;              // rows i per group
  const int GI = (I + rpg - 1) / rpg;     // groups per slot
  const int ngroups = T * k * GI;
  const int groups_lo = ngroups / nb, extra = ngroups % nb;
  const int g_begin = bid * groups_lo + (bid < extra ? bid : extra);
  const int g_end = g_begin + groups_lo + (bid < extra ? 1 : 0);
  if (g_begin >= g_end) {
    issued();
    return;
  }
  const int wave_groups = g_end - g_begin > wave ? (g_end - g_begin - wave + NW - 1) / NW : 0;
  const int iters = (nch + LPR - 1) >> lpr_log2;
  const int blk_shift = __builtin_ctz((unsigned)a.block) - 5;
  const uint32_t rb = (uint32_t)a.fc1_row_bytes;
  const uint32_t zrb = (uint32_t)a.fc1_zp_row_bytes;
  const uint32_t erows = 2u * (uint32_t)I;  // W1 rows per expert

  // fetch cursor: group, item, and the expert's buffers and rows of that group
  int fgrp = g_begin + wave, fit = 0;
  __amdgpu_buffer_rsrc_t rW, rS, rZ;
  uint32_t frow[NR];
  auto set_group = [&](int grp) {
    // Past the wave's own groups (the ring's run-ahead at the end of its work, or a
    // wave with none) the buffers get range 0: those loads return 0 and move no data.
    // (The groups that follow belong to the next work-group, on another XCD.)
    const uint32_t on = grp < g_end ? 1u : 0u;
    const int gg = grp < ngroups ? grp : ngroups - 1;
    const int sl = gg / GI;
    const int gi = gg - sl * GI;
    const int e = clamp_expert(a.ids[sl], a.E);
    rW = make_rsrc(a.fc1.W + (size_t)e * erows * rb, on * erows * rb);
    rS = make_rsrc((const uint16_t*)a.fc1.scales + (size_t)e * erows * nblk, on * erows * (uint32_t)nblk * 2u);
    if constexpr (ZK) rZ = make_rsrc(a.fc1.zp + (size_t)e * erows * zrb, on * erows * zrb);
#pragma unroll
    for (int r = 0; r < RI; ++r) {
      const int i = gi * rpg + r * SUBS + sub;
      const uint32_t ic = (uint32_t)(i < I ? i : I - 1);
      frow[2 * r] = ic;
      frow[2 * r + 1] = ic + (uint32_t)I;
    }
  };
  auto fetch = [&](MoeItem<NR>& b) {
    int c = fit * LPR + lp;
    c = c < nch ? c : nch - 1;
    const int blk = c >> blk_shift;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)(frow[r] * rb + (uint32_t)c * 16u), 0, 0);
      b.w[r] = make_uint4(v[0], v[1], v[2], v[3]);
      b.s[r] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(
                                                 rS, (int)((frow[r] * (uint32_t)nblk + (uint32_t)blk) * 2u), 0, 0));
      if constexpr (ZK)
        b.z[r] = __builtin_amdgcn_raw_buffer_load_b8(rZ, (int)(frow[r] * zrb + (uint32_t)(blk >> 1)), 0, 0);
      else
        b.z[r] = 0x88u;
    }
    if (++fit == iters) {
      fit = 0;
      fgrp += NW;
      set_group(fgrp);
    }
  };
  auto token_of = [&](int grp) { return ((grp < ngroups ? grp : ngroups - 1) / GI) / k; };

  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
  int cgrp = g_begin + wave, cit = 0, ct = token_of(cgrp);
  auto step = [&](const MoeItem<NR>& cb, MoeItem<NR>& nxt, bool live) {
    fetch(nxt);
    const int c = cit * LPR + lp;
    const bool cv = live && c < nch;
    const int cc = c < nch ? c : nch - 1;
    const int blk = cc >> blk_shift;
    if constexpr (INT8) {
      const uint32_t* xqt = xq + (size_t)ct * (H / 4);
      const uint4 q0 = *(const uint4*)(xqt + cc * 8);
      const uint4 q1 = *(const uint4*)(xqt + cc * 8 + 4);
      const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const float sx = xs[ct * (H / 32) + cc];
      const int sum = xsum[ct * (H / 32) + cc];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int dotv = dot_chunk_u4_i8(cb.w[r], qq);
        const int zp = (int)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
        const float nv = fmaf((float)cb.s[r] * sx, (float)(dotv - zp * sum), acc[r]);
        acc[r] = cv ? nv : acc[r];
      }
    } else {
      const uint32_t* xp = xh + ((size_t)ct * nch + cc) * kPairStride;
      uint32_t xa[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = load_pairs(xp + 4 * q);
        xa[4 * q] = v.x; xa[4 * q + 1] = v.y; xa[4 * q + 2] = v.z; xa[4 * q + 3] = v.w;
      }
      const float sac = sa[ct * nch + cc];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float pr = dot_chunk_u4(cb.w[r], xa);
        const float zp = (float)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
        const float nv = fmaf((float)cb.s[r], fmaf(-zp, sac, pr), acc[r]);
        acc[r] = cv ? nv : acc[r];
      }
    }
    if (live && cit == iters - 1) {
      // group complete: fixed-order combination of the LPR lane partials
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = group_sum(acc[r], LPR);
      if (lp == 0) {
#pragma unroll
        for (int r = 0; r < RI; ++r) {
          const int lr = (cgrp - g_begin) * rpg + r * SUBS + sub;
          outs[2 * lr] = acc[2 * r];
          outs[2 * lr + 1] = acc[2 * r + 1];
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
    }
    if (++cit == iters) {
      cit = 0;
      cgrp += NW;
      ct = token_of(cgrp);
    }
  };

  // the activations' loads go out first, then the first weights, which travel while
  // the activations are converted
  MoeItem<NR> buf[D];
  set_group(fgrp);
  if constexpr (INT8) {
    // every token's x quantized into LDS (work-group 0 keeps a copy in scratch)
    stage_i8_first<0>(a.X, T * H, xq, xs, xsum, bid == 0 ? a.xq_out : nullptr, bid == 0 ? a.xs_out : nullptr, [&] {
#pragma unroll
      for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
      issued();
    });
  } else {
    stage_h16_first(a.X, T, (int)a.H, nch, xh, sa, [&] {
#pragma unroll
      for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
      issued();
    });
  }
  const int total = wave_groups * iters;
  for (int base = 0; base < total; base += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) step(buf[i], buf[(i + D - 1) % D], base + i < total);
  }
  __syncthreads();
  // bias and SwiGLU of every row of the work-group's groups
  const int nloc = (g_end - g_begin) * rpg;
  for (int q = threadIdx.x; q < nloc; q += blockDim.x) {
    const int grp = g_begin + q / rpg;
    const int sl = grp / GI;
    const int i = (grp - sl * GI) * rpg + (q - (q / rpg) * rpg);
    if (i >= I) continue;
    float g = outs[2 * q], u = outs[2 * q + 1];
    if (a.fc1.bias) {
      const int e = clamp_expert(a.ids[sl], a.E);
      const uint16_t* bb = a.fc1.bias + (int64_t)e * 2 * a.I;
      g += f16_to_f32(bb[i]);
      u += f16_to_f32(bb[i + a.I]);
    }
    const float hv = g / (1.0f + expf(-g)) * u;
    if constexpr (COH)
      __hip_atomic_store(a.h + (int64_t)sl * a.I + i, f32_to_f16(hv), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      a.h[(int64_t)sl * a.I + i] = f32_to_f16(hv);
  }
}

template <int RI, int ZK, int INT8>
__global__ __launch_bounds__(kMoeStreamThreads) void qmoe_fc1_stream_kernel(QmoeArgs a) {
  extern __shared__ uint32_t smem[];
  fc1_stream_body<RI, ZK, false, INT8 != 0>(a, (int)blockIdx.x, (int)gridDim.x, smem, [] {});
}


// fc2 write-out: y = sum_j w_j * (z_j + b2) in slot order, one rounding to fp16, for
// every row of the work-group's groups [g_begin, g_end) (outs[local row][k]: the row
// sums z_j without bias).
__device__ __forceinline__ void fc2_write_out(const QmoeArgs& a, int g_begin, int g_end, int rpg, int GN,
                                              const float* outs) {
  __syncthreads();
  const int k = a.k;
  const int H = (int)a.H;
  const int nloc = (g_end - g_begin) * rpg;
  for (int q = threadIdx.x; q < nloc; q += blockDim.x) {
    const int grp = g_begin + q / rpg;
    const int t = grp / GN;
    const int n = (grp - t * GN) * rpg + (q - (q / rpg) * rpg);
    if (n >= H) continue;
    float y = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int e = clamp_expert(a.ids[t * k + j], a.E);
      const float z = outs[q * k + j] + (a.fc2.bias ? f16_to_f32(a.fc2.bias[(int64_t)e * a.H + n]) : 0.0f);
      y = fmaf(a.rw[t * k + j], z, y);
    }
    a.Y[(int64_t)t * a.H + n] = f32_to_f16(y);
  }
}

// FUSED: h was written earlier in the same launch by other work-groups: the first
// weight loads are issued, then `wait()` (every work-group's h is complete), then h is
// staged with device-coherent loads.
template <int R, int ZK, bool FUSED, typename Wait, bool INT8 = false>
__device__ __forceinline__ void fc2_stream_body(const QmoeArgs& a, int bid, int nb, uint32_t* smem, Wait&& wait) {
  constexpr int NW = kMoeStreamThreads / 64;
  constexpr int D = kFc2Depth;
  const int T = (int)a.T;
  const int k = a.k;
  const int H = (int)a.H;
  const int nch = (int)a.fc2_chunks;
  const int nblk = (int)a.fc2_nblk;
  const int I = (int)a.I;
  uint32_t* hh = smem;                         // fp: [T * k][nch][kPairStride] fp16 pairs
  float* sa = (float*)(hh + (size_t)T * k * nch * kPairStride);  // fp: [T * k][nch]
  uint32_t* hq = smem;                         // int8: [T * k][I / 4] permuted codes
  float* hs = (float*)(smem + (size_t)T * k * I / 4);  // int8: [T * k][I / 32] scales
  int* hsum = (int*)(hs + (size_t)T * k * I / 32);     // int8: [T * k][I / 32] code sums
  float* outs = INT8 ? (float*)(hsum + (size_t)T * k * I / 32) : sa + (size_t)T * k * nch;  // [local rows][k]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lpr_log2 = a.fc2_lpr_log2;
  const int LPR = 1 << lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> lpr_log2;
  const int SUBS = 64 >> lpr_log2;
  const int rpg = SUBS * R;               // rows n per group
  const int GN = (H + rpg - 1) / rpg;     // groups per token
  const int ngroups = T * GN;
  const int groups_lo = ngroups / nb, extra = ngroups % nb;
  const int g_begin = bid * groups_lo + (bid < extra ? bid : extra);
  const int g_end = g_begin + groups_lo + (bid < extra ? 1 : 0);
  if (g_begin >= g_end) return;
  // the work-group's units are (group, slot) pairs, unit u = (g_begin + u / k, u % k);
  // wave w takes units w, w + NW, ... (the slot sums are combined at the write-out)
  const int nunits = (g_end - g_begin) * k;
  const int wave_units = nunits > wave ? (nunits - wave + NW - 1) / NW : 0;
  const int iters = (nch + LPR - 1) >> lpr_log2;
  const int blk_shift = __builtin_ctz((unsigned)a.block) - 5;
  const uint32_t rb = (uint32_t)a.fc2_row_bytes;
  const uint32_t zrb = (uint32_t)a.fc2_zp_row_bytes;
  const uint32_t erows = (uint32_t)H;  // W2 rows per expert

  // fetch cursor: unit and item, and the unit's expert buffers and rows
  int fu = wave, fit = 0;
  __amdgpu_buffer_rsrc_t rW, rS, rZ;
  uint32_t frow[R];
  auto set_unit = [&](int u) {
    // past the wave's own units the buffers get range 0 (loads return 0, move no data)
    const uint32_t on = u < nunits ? 1u : 0u;
    const int uu = u < nunits ? u : nunits - 1;
    const int grp = g_begin + uu / k;
    const int j = uu - (uu / k) * k;
    const int t = grp / GN;
    const int gn = grp - t * GN;
    const int e = clamp_expert(a.ids[t * k + j], a.E);
    rW = make_rsrc(a.fc2.W + (size_t)e * erows * rb, on * erows * rb);
    rS = make_rsrc((const uint16_t*)a.fc2.scales + (size_t)e * erows * nblk, on * erows * (uint32_t)nblk * 2u);
    if constexpr (ZK) rZ = make_rsrc(a.fc2.zp + (size_t)e * erows * zrb, on * erows * zrb);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = gn * rpg + r * SUBS + sub;
      frow[r] = (uint32_t)(n < H ? n : H - 1);
    }
  };
  auto fetch = [&](MoeItem<R>& b) {
    int c = fit * LPR + lp;
    c = c < nch ? c : nch - 1;
    const int blk = c >> blk_shift;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)(frow[r] * rb + (uint32_t)c * 16u), 0, 0);
      b.w[r] = make_uint4(v[0], v[1], v[2], v[3]);
      b.s[r] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(
                                                 rS, (int)((frow[r] * (uint32_t)nblk + (uint32_t)blk) * 2u), 0, 0));
      if constexpr (ZK)
        b.z[r] = __builtin_amdgcn_raw_buffer_load_b8(rZ, (int)(frow[r] * zrb + (uint32_t)(blk >> 1)), 0, 0);
      else
        b.z[r] = 0x88u;
    }
    if (++fit == iters) {
      fit = 0;
      fu += NW;
      set_unit(fu);
    }
  };
  // compute cursor: unit cu (local row base and slot), item cit
  int cu = wave, cit = 0, c_lr = 0, c_j = 0, c_hrow = 0;
  auto set_cunit = [&](int u) {
    const int uu = u < nunits ? u : nunits - 1;
    const int grp = g_begin + uu / k;
    c_j = uu - (uu / k) * k;
    c_lr = (grp - g_begin) * rpg;
    c_hrow = (grp / GN) * k + c_j;  // row t * k + j of the staged h
  };
  set_cunit(cu);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  auto step = [&](const MoeItem<R>& cb, MoeItem<R>& nxt, bool live) {
    fetch(nxt);
    const int c = cit * LPR + lp;
    const bool cv = live && c < nch;
    const int cc = c < nch ? c : nch - 1;
    const int blk = cc >> blk_shift;
    if constexpr (INT8) {
      const uint32_t* qg = hq + ((size_t)c_hrow * I + cc * 32) / 4;
      const uint4 q0 = *(const uint4*)(qg);
      const uint4 q1 = *(const uint4*)(qg + 4);
      const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const int gi = (c_hrow * I + cc * 32) / 32;
      const float sx = hs[gi];
      const int sum = hsum[gi];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int dotv = dot_chunk_u4_i8(cb.w[r], qq);
        const int zp = (int)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
        const float nv = fmaf((float)cb.s[r] * sx, (float)(dotv - zp * sum), acc[r]);
        acc[r] = cv ? nv : acc[r];
      }
    } else {
      const uint32_t* xp = hh + ((size_t)c_hrow * nch + cc) * kPairStride;
      uint32_t xa[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = load_pairs(xp + 4 * q);
        xa[4 * q] = v.x; xa[4 * q + 1] = v.y; xa[4 * q + 2] = v.z; xa[4 * q + 3] = v.w;
      }
      const float sac = sa[c_hrow * nch + cc];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pr = dot_chunk_u4(cb.w[r], xa);
        const float zp = (float)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
        const float nv = fmaf((float)cb.s[r], fmaf(-zp, sac, pr), acc[r]);
        acc[r] = cv ? nv : acc[r];
      }
    }
    if (live && cit == iters - 1) {
      // unit complete: fixed-order combination of the lane partials of its slot
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = group_sum(acc[r], LPR);
      if (lp == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) outs[(c_lr + r * SUBS + sub) * k + c_j] = acc[r];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    }
    if (++cit == iters) {
      cit = 0;
      cu += NW;
      set_cunit(cu);
    }
  };

  // the activations' loads go out first, then the first weights, which travel while
  // the activations are converted
  MoeItem<R> buf[D];
  set_unit(fu);
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
    wait();
    if constexpr (INT8)
      stage_i8_first<kDeviceCoherent>(a.h, T * k * I, hq, hs, hsum, bid == 0 ? a.hq_out : nullptr,
                                      bid == 0 ? a.hs_out : nullptr, [] {});
    else
      stage_h16_first<kDeviceCoherent>(a.h, T * k, (int)a.I, nch, hh, sa, [] {});
  } else if constexpr (INT8) {
    // the codes and scales of every slot's h (quantized once per call into scratch)
#pragma unroll
    for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
    stage_i8(a.hq_out, a.hs_out, T * k * I, hq, hs, hsum);
  } else {
    stage_h16_first(a.h, T * k, (int)a.I, nch, hh, sa, [&] {
#pragma unroll
      for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
    });
  }
  const int total = wave_units * iters;
  for (int base = 0; base < total; base += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) step(buf[i], buf[(i + D - 1) % D], base + i < total);
  }
  fc2_write_out(a, g_begin, g_end, rpg, GN, outs);
}

template <int R, int ZK, int INT8>
__global__ __launch_bounds__(kMoeStreamThreads) void qmoe_fc2_stream_kernel(QmoeArgs a) {
  extern __shared__ uint32_t smem[];
  auto no_wait = [] {};
  fc2_stream_body<R, ZK, false, decltype(no_wait)&, INT8 != 0>(a, (int)blockIdx.x, (int)gridDim.x, smem, no_wait);
}


// ---- fc1 reading each expert's rows once per call (fp mode, 1 < T <= kDedupeMaxT) ------
//
// The slots routed to one expert share every load of its rows.  The row groups walk the
// distinct experts of the call (in order of first use), each with the list of its slots
// in slot order (split into units of at most kDedupeMaxT slots).  A lane loads each
// chunk of its rows once and runs the per-slot chunk arithmetic of the stream form for
// every slot of the unit, so every slot's h has the bits of the per-slot forms.
constexpr int kDedupeMaxT = 8;                 // slots per expert at most (one per token)
// LDS ints: expert and first use of each slot, the slot list, the start and expert of
// each distinct expert, the start, count and expert of each unit, the unit count and
// a split flag
constexpr int kDedupeInts = 8 * kMoeSortSlots + 3;

template <int RI, int ZK>
__global__ __launch_bounds__(kMoeStreamThreads) void qmoe_fc1_dedupe_kernel(QmoeArgs a) {
  constexpr int NR = 2 * RI;  // per row i: the g row and the u row
  constexpr int NW = kMoeStreamThreads / 64;
  constexpr int D = RI == 1 ? 4 : 3;
  constexpr int MS = kDedupeMaxT;
  extern __shared__ uint32_t smem[];
  const int T = (int)a.T;
  const int k = a.k;
  const int I = (int)a.I;
  const int S = T * k;
  const int nch = (int)a.fc1_chunks;
  const int nblk = (int)a.fc1_nblk;
  uint32_t* xh = smem;                         // [T][nch][kPairStride] fp16 pairs
  float* sa = (float*)(xh + (size_t)T * nch * kPairStride);  // [T][nch]
  int* eid = (int*)(sa + (size_t)T * nch);     // [S] expert of each slot
  int* first = eid + kMoeSortSlots;            // [S] first slot with the same expert
  int* ulist = first + kMoeSortSlots;          // [S] slots grouped by expert
  int* ustart = ulist + kMoeSortSlots;         // [U + 1] start of each expert's slots
  int* uexp = ustart + kMoeSortSlots + 1;      // [U] the distinct experts
  int* vstart = uexp + kMoeSortSlots;          // [V] units: start in the slot list,
  int* vcnt = vstart + kMoeSortSlots;          //     slot count (<= MS),
  int* vexp = vcnt + kMoeSortSlots;            //     expert
  int* vnum = vexp + kMoeSortSlots;            // [2] V, and whether any expert needs splitting
  float* outs = (float*)(eid + kDedupeInts);   // [local rows][MS][2]: g and u sums per slot

  // distinct experts in order of first use and their slots, in three passes
  for (int s = threadIdx.x; s < S; s += blockDim.x) eid[s] = clamp_expert(a.ids[s], a.E);
  if (threadIdx.x == 0) vnum[0] = 0, vnum[1] = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = eid[s];
    int f = s;
#pragma unroll 16
    for (int s2 = 0; s2 < S; ++s2) f = (s2 < f && eid[s2] == e) ? s2 : f;
    first[s] = f;
  }
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int f = first[s];
    int pos = 0, u = 0, cnt = 0;
#pragma unroll 16
    for (int s2 = 0; s2 < S; ++s2) {
      const int f2 = first[s2];
      pos += (f2 < f || (f2 == f && s2 < s)) ? 1 : 0;
      u += (s2 < f && f2 == s2) ? 1 : 0;
      cnt += f2 == f ? 1 : 0;
    }
    ulist[pos] = s;
    if (f == s) {
      ustart[u] = pos;
      uexp[u] = eid[s];
      vstart[u] = pos;
      vcnt[u] = cnt;
      vexp[u] = eid[s];
      atomicAdd(&vnum[0], 1);
      if (cnt > MS) vnum[1] = 1;  // an expert repeated inside a token
    }
  }
  __syncthreads();
  // units of at most MS slots: normally one per distinct expert; a call that repeats
  // an expert inside a token has that expert's slots split (one thread, rare)
  if (vnum[1] != 0 && threadIdx.x == 0) {
    const int U = vnum[0];
    ustart[U] = S;
    int V = 0;
    for (int u = 0; u < U; ++u) {
      const int cnt = ustart[u + 1] - ustart[u];
      for (int off = 0; off < cnt; off += MS) {
        vstart[V] = ustart[u] + off;
        vcnt[V] = cnt - off < MS ? cnt - off : MS;
        vexp[V] = uexp[u];
        ++V;
      }
    }
    vnum[0] = V;
  }
  __syncthreads();
  const int V = vnum[0];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lpr_log2 = a.fc1_lpr_log2;
  const int LPR = 1 << lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> lpr_log2;
  const int SUBS = 64 >> lpr_log2;
  const int rpg = SUBS * RI;              // rows i per group
  const int GI = (I + rpg - 1) / rpg;     // groups per unit
  const int ngroups = V * GI;
  const int nb = (int)gridDim.x, bid = (int)blockIdx.x;
  const int groups_lo = ngroups / nb, extra = ngroups % nb;
  const int g_begin = bid * groups_lo + (bid < extra ? bid : extra);
  const int g_end = g_begin + groups_lo + (bid < extra ? 1 : 0);
  if (g_begin >= g_end) return;
  const int wave_groups = g_end - g_begin > wave ? (g_end - g_begin - wave + NW - 1) / NW : 0;
  const int iters = (nch + LPR - 1) >> lpr_log2;
  const int blk_shift = __builtin_ctz((unsigned)a.block) - 5;
  const uint32_t rb = (uint32_t)a.fc1_row_bytes;
  const uint32_t zrb = (uint32_t)a.fc1_zp_row_bytes;
  const uint32_t erows = 2u * (uint32_t)I;

  int fgrp = g_begin + wave, fit = 0;
  __amdgpu_buffer_rsrc_t rW, rS, rZ;
  uint32_t frow[NR];
  auto set_group = [&](int grp) {
    // past the wave's own groups the buffers get range 0 (loads return 0, move no data)
    const uint32_t on = grp < g_end ? 1u : 0u;
    const int gg = grp < ngroups ? grp : ngroups - 1;
    const int v = gg / GI;
    const int gi = gg - v * GI;
    const int e = vexp[v];
    rW = make_rsrc(a.fc1.W + (size_t)e * erows * rb, on * erows * rb);
    rS = make_rsrc((const uint16_t*)a.fc1.scales + (size_t)e * erows * nblk, on * erows * (uint32_t)nblk * 2u);
    if constexpr (ZK) rZ = make_rsrc(a.fc1.zp + (size_t)e * erows * zrb, on * erows * zrb);
#pragma unroll
    for (int r = 0; r < RI; ++r) {
      const int i = gi * rpg + r * SUBS + sub;
      const uint32_t ic = (uint32_t)(i < I ? i : I - 1);
      frow[2 * r] = ic;
      frow[2 * r + 1] = ic + (uint32_t)I;
    }
  };
  auto fetch = [&](MoeItem<NR>& b) {
    int c = fit * LPR + lp;
    c = c < nch ? c : nch - 1;
    const int blk = c >> blk_shift;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)(frow[r] * rb + (uint32_t)c * 16u), 0, 0);
      b.w[r] = make_uint4(v[0], v[1], v[2], v[3]);
      b.s[r] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(
                                                 rS, (int)((frow[r] * (uint32_t)nblk + (uint32_t)blk) * 2u), 0, 0));
      if constexpr (ZK)
        b.z[r] = __builtin_amdgcn_raw_buffer_load_b8(rZ, (int)(frow[r] * zrb + (uint32_t)(blk >> 1)), 0, 0);
      else
        b.z[r] = 0x88u;
    }
    if (++fit == iters) {
      fit = 0;
      fgrp += NW;
      set_group(fgrp);
    }
  };

  // compute cursor: group, item, and the tokens of the group's slots
  int cgrp = g_begin + wave, cit = 0, ccnt = 0;
  int ctok[MS];
  auto set_cgroup = [&](int grp) {
    const int gg = grp < ngroups ? grp : ngroups - 1;
    const int v = gg / GI;
    const int s0 = vstart[v];
    ccnt = vcnt[v];
#pragma unroll
    for (int q = 0; q < MS; ++q) ctok[q] = ulist[s0 + (q < ccnt ? q : 0)] / k;
  };
  float acc[MS][NR];
#pragma unroll
  for (int q = 0; q < MS; ++q)
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[q][r] = 0.0f;
  auto step = [&](const MoeItem<NR>& cb, MoeItem<NR>& nxt, bool live) {
    fetch(nxt);
    const int c = cit * LPR + lp;
    const bool cv = live && c < nch;
    const int cc = c < nch ? c : nch - 1;
    const int blk = cc >> blk_shift;
#pragma unroll
    for (int q = 0; q < MS; ++q) {
      if (q < ccnt) {
        const uint32_t* xp = xh + ((size_t)ctok[q] * nch + cc) * kPairStride;
        uint32_t xa[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 v = load_pairs(xp + 4 * j);
          xa[4 * j] = v.x; xa[4 * j + 1] = v.y; xa[4 * j + 2] = v.z; xa[4 * j + 3] = v.w;
        }
        const float sac = sa[ctok[q] * nch + cc];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float pr = dot_chunk_u4(cb.w[r], xa);
          const float zp = (float)((cb.z[r] >> ((blk & 1) * 4)) & 0xfu);
          const float nv = fmaf((float)cb.s[r], fmaf(-zp, sac, pr), acc[q][r]);
          acc[q][r] = cv ? nv : acc[q][r];
        }
      }
    }
    if (live && cit == iters - 1) {
#pragma unroll
      for (int q = 0; q < MS; ++q) {
        if (q < ccnt) {
#pragma unroll
          for (int r = 0; r < RI; ++r) {
            const float g = group_sum(acc[q][2 * r], LPR);
            const float u = group_sum(acc[q][2 * r + 1], LPR);
            if (lp == 0) {
              const int lr = (cgrp - g_begin) * rpg + r * SUBS + sub;
              outs[(lr * MS + q) * 2] = g;
              outs[(lr * MS + q) * 2 + 1] = u;
            }
          }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[q][r] = 0.0f;
      }
    }
    if (++cit == iters) {
      cit = 0;
      cgrp += NW;
      set_cgroup(cgrp);
    }
  };

  MoeItem<NR> buf[D];
  set_group(fgrp);
  set_cgroup(cgrp);
  stage_h16_first(a.X, T, (int)a.H, nch, xh, sa, [&] {
#pragma unroll
    for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
  });
  const int total = wave_groups * iters;
  for (int base = 0; base < total; base += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) step(buf[i], buf[(i + D - 1) % D], base + i < total);
  }
  __syncthreads();
  // bias and SwiGLU for every slot of every row of the work-group's groups
  const int nloc = (g_end - g_begin) * rpg;
  for (int q2 = threadIdx.x; q2 < nloc * MS; q2 += blockDim.x) {
    const int lr = q2 / MS, q = q2 - lr * MS;
    const int grp = g_begin + lr / rpg;
    const int v = grp / GI;
    const int i = (grp - v * GI) * rpg + (lr - (lr / rpg) * rpg);
    if (i >= I || q >= vcnt[v]) continue;
    const int sl = ulist[vstart[v] + q];
    float g = outs[(lr * MS + q) * 2], uu = outs[(lr * MS + q) * 2 + 1];
    if (a.fc1.bias) {
      const uint16_t* bb = a.fc1.bias + (int64_t)vexp[v] * 2 * a.I;
      g += f16_to_f32(bb[i]);
      uu += f16_to_f32(bb[i + a.I]);
    }
    const float hv = g / (1.0f + expf(-g)) * uu;
    a.h[(int64_t)sl * a.I + i] = f32_to_f16(hv);
  }
}

// ---- single-launch form ------------------------------------------------------------
//
// fc1, SwiGLU, fc2 and the combine in one launch of the persistent forms above: one
// grid of work-groups, all resident at once (the grid is the occupancy of this kernel
// times the compute units).  Each work-group runs its even share of the fc1 row
// groups, writes its h rows with device-coherent stores, waits for them to complete
// and counts itself arrived.  It then issues the first weight loads of its fc2 share,
// waits until every work-group has arrived, stages h with device-coherent loads (int8
// mode: and quantizes it) and runs its fc2 share (all k slots of its rows, combined in
// slot order).  The per-row arithmetic is that of the two-kernel forms, so every form
// gives the same bits.
//
// The wait is sense-reversing and counts in two levels, spread over slots of 256 bytes
// so that arrivals and polls do not queue on one address: work-group b belongs to slot
// 1 + b % kQmoeSyncSubs, which holds a sub-counter and a copy of the phase.  Each
// work-group reads its slot's phase when it starts and adds its arrival to its slot's
// sub-counter; the add returns the count before it, so the last arrival of a slot knows
// it is last, returns the sub-counter to zero and adds one to the top counter (slot 0);
// the last of those returns the top counter to zero and flips every slot's phase, and
// every other work-group waits for its slot's phase to change.  Nothing is left to do
// at exit, and the next call finds every counter at zero and every phase equal.
//
// Ordering across the XCDs (each with its own L2) without whole-cache operations: the
// h stores are agent-scope atomic stores, which write through the L2; the work-group
// waits until every one of them is acknowledged (s_waitcnt) before its agent-scope
// arrival add, so a count that includes it implies its h is in memory; a counter's
// last add returns only once every earlier add to it is performed, and the top add of
// a sub-counter's last arrival is issued only after its sub-counter add returned.  A waiting
// work-group reads the phase with agent-scope loads (which miss the L2) and only after
// it has seen the flip issues its h loads, which are device-coherent (they also miss
// the L2) and are ordered after the poll by the work-group barrier.  A release/acquire
// pair would add an L2 write-back per arrival and an L2 invalidation per waiter,
// several microseconds per call, to order data that never enters the L2.

// a wait gives up after 1 s of the 100 MHz real-time counter and raises the error word
constexpr uint64_t kSpinLimitTicks = 100000000ull;

// arrival: the caller has waited for every h store of the work-group (write-through
// agent-scope stores) to be acknowledged; returns the count before this arrival
__device__ __forceinline__ uint32_t sync_arrive(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t sync_load(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sync_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int RI, int R, int ZK1, int ZK2, int INT8>
__global__ __launch_bounds__(kMoeStreamThreads) void qmoe_fused_kernel(QmoeArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t gave_up;
  uint32_t* sync = a.sync;
  const int nb = (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  if (threadIdx.x == 0) gave_up = 0u;
  // this work-group's sync slot and the phase before this call (the flip needs every
  // work-group's arrival, this one's too)
  uint32_t* slot = sync + (size_t)(1 + bid % kQmoeSyncSubs) * kQmoeSyncSlotWords;
  const uint32_t phase = threadIdx.x == 0 ? sync_load(&slot[1]) : 0u;
  fc1_stream_body<RI, ZK1, true, INT8 != 0>(a, bid, nb, smem, [] {});
  // every wave's h stores (and the phase load) have completed before the work-group
  // counts itself arrived
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bool last = false;
  if (threadIdx.x == 0) {
    const int sub = bid % kQmoeSyncSubs;
    const int nsub = nb < kQmoeSyncSubs ? nb : kQmoeSyncSubs;  // slots in use
    const uint32_t in_sub = (uint32_t)(nb / kQmoeSyncSubs + (sub < nb % kQmoeSyncSubs ? 1 : 0));
    if (sync_arrive(&slot[0]) == in_sub - 1u) {
      sync_store(&slot[0], 0u);
      if (sync_arrive(&sync[0]) == (uint32_t)nsub - 1u) {
        last = true;
        sync_store(&sync[0], 0u);
        for (int i = 1; i <= kQmoeSyncSubs; ++i) sync_store(&sync[(size_t)i * kQmoeSyncSlotWords + 1], phase ^ 1u);
      }
    }
  }
  auto wait = [&] {
    if (threadIdx.x == 0 && !last) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (sync_load(&slot[1]) == phase) {
        __builtin_amdgcn_s_sleep(2);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimitTicks) {
          sync_store(&sync[2], 1u);
          gave_up = 1u;
          break;
        }
      }
    }
    __syncthreads();
  };
  fc2_stream_body<R, ZK2, true, decltype(wait)&, INT8 != 0>(a, bid, nb, smem, wait);
  __syncthreads();
  if (gave_up) {
    // a wait that gave up leaves the output invalid: it is filled with fp16 NaN (after
    // this work-group's own rows were written, so those rows are NaN at the end)
    for (int64_t i = threadIdx.x; i < a.T * a.H; i += kMoeStreamThreads) a.Y[i] = 0x7E00u;
  }
}

// ---- launch ---------------------------------------------------------------------

size_t qmoe_fc1_lds_bytes(const QmoeArgs& a) {
  if (a.mode == QMOE_INT8_ACT) return (size_t)a.H + (size_t)(a.H / 32) * 8;
  return (size_t)a.fc1_chunks * kStagedWords * sizeof(uint32_t);
}
size_t qmoe_fc2_lds_bytes(const QmoeArgs& a) {
  if (a.mode == QMOE_INT8_ACT) return (size_t)(a.k * a.I) + (size_t)(a.k * a.I / 32) * 8;
  return (size_t)a.k * a.fc2_chunks * kStagedWords * sizeof(uint32_t);
}

// Allow more than 64 KB of dynamic LDS for a kernel: up to the 150 KB the launch plans
// use, which leaves room for a kernel's few bytes of static LDS within the 160 KB.
template <typename Kern>
static void allow_lds(Kern k, size_t lds) {
  if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
}

// Work-groups of `kern` with `lds` bytes of dynamic LDS resident on one compute unit
// (cached per kernel and size).
template <typename Kern>
static int moe_resident_per_cu(Kern kern, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<const void*, size_t>, int> cache;
  const auto key = std::make_pair((const void*)kern, lds);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  allow_lds(kern, lds);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kMoeStreamThreads, lds) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  cache[key] = n;
  return n;
}

// Grid and LDS of a persistent form: one work-group per resident slot (at most one
// per group), `fixed` bytes of staged activations plus `per_group` bytes of row sums
// for each group of the work-group.  Returns false when it does not fit in LDS.
// `cap` limits the work-groups per compute unit (fewer, longer work-groups stage the
// activations fewer times).
template <typename Kern>
static bool moe_stream_plan(Kern kern, int64_t ngroups, size_t fixed, size_t per_group, int num_cus, int cap,
                            int64_t* grid, size_t* lds) {
  constexpr size_t kMaxStreamLds = 150 * 1024;
  if (ngroups < 1 || fixed + per_group > kMaxStreamLds) return false;
  int per_cu = moe_resident_per_cu(kern, fixed + per_group);
  if (per_cu > cap) per_cu = cap;
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t slots = (int64_t)(num_cus > 0 ? num_cus : 256) * per_cu;
    *grid = slots < ngroups ? slots : ngroups;
    *lds = fixed + (size_t)((ngroups + *grid - 1) / *grid) * per_group;
    if (*lds > kMaxStreamLds) return false;
    const int again = moe_resident_per_cu(kern, *lds);
    if (again >= per_cu) break;
    per_cu = again;
  }
  return true;
}

template <int RI, int ZK, int INT8>
static bool launch_fc1_stream(const QmoeArgs& a, int cap, hipStream_t st) {
  auto kern = qmoe_fc1_stream_kernel<RI, ZK, INT8>;
  // one expert's W1, scales and zero points are addressed with 32-bit offsets
  const int64_t erows = 2 * a.I;
  if (erows * a.fc1_row_bytes >= (1LL << 31) || erows * a.fc1_nblk * 2 >= (1LL << 31)) return false;
  const int64_t rpg = (64 >> a.fc1_lpr_log2) * RI;
  const int64_t ngroups = a.T * a.k * ((a.I + rpg - 1) / rpg);
  // staged activations: fp32 values and chunk sums, or int8 codes, scales and code sums
  const size_t fixed = INT8 ? (size_t)a.T * ((size_t)a.H + (size_t)(a.H / 32) * 8)
                            : (size_t)a.T * a.fc1_chunks * kStagedWords * sizeof(uint32_t);
  int64_t grid = 0;
  size_t lds = 0;
  if (!moe_stream_plan(kern, ngroups, fixed, (size_t)rpg * 2 * sizeof(float), a.num_cus, cap, &grid, &lds))
    return false;
  allow_lds(kern, lds);
  launch(kern, dim3((unsigned)grid), dim3(kMoeStreamThreads), lds, st, a);
  return true;
}

template <int R, int ZK, int INT8>
static bool launch_fc2_stream(const QmoeArgs& a, int cap, hipStream_t st) {
  auto kern = qmoe_fc2_stream_kernel<R, ZK, INT8>;
  if (a.H * a.fc2_row_bytes >= (1LL << 31) || a.H * a.fc2_nblk * 2 >= (1LL << 31)) return false;
  const int64_t rpg = (64 >> a.fc2_lpr_log2) * R;
  const int64_t ngroups = a.T * ((a.H + rpg - 1) / rpg);
  const size_t fixed = INT8 ? (size_t)a.T * a.k * ((size_t)a.I + (size_t)(a.I / 32) * 8)
                            : (size_t)a.T * a.k * a.fc2_chunks * kStagedWords * sizeof(uint32_t);
  int64_t grid = 0;
  size_t lds = 0;
  if (!moe_stream_plan(kern, ngroups, fixed, (size_t)rpg * a.k * sizeof(float), a.num_cus, cap, &grid, &lds))
    return false;
  allow_lds(kern, lds);
  launch(kern, dim3((unsigned)grid), dim3(kMoeStreamThreads), lds, st, a);
  return true;
}


// LDS of the single-launch form at `grid` work-groups: the larger of the fc1 and fc2
// phases' staged activations and row sums.  0 when the shape does not suit the form
// (32-bit offsets).
static size_t fused_lds(const QmoeArgs& a, int R2, int64_t grid) {
  const bool i8 = a.mode == QMOE_INT8_ACT;
  const int64_t r1 = 2 * a.I, r2 = a.H;
  // one expert's weights, scales and zero points are addressed with 32-bit offsets
  if (r1 * a.fc1_row_bytes >= (1LL << 31) || r1 * a.fc1_nblk * 2 >= (1LL << 31)) return 0;
  if (r2 * a.fc2_row_bytes >= (1LL << 31) || r2 * a.fc2_nblk * 2 >= (1LL << 31)) return 0;
  const int64_t rpg1 = (64 >> a.fc1_lpr_log2) * 2, rpg2 = (64 >> a.fc2_lpr_log2) * R2;
  const int64_t ng1 = a.T * a.k * ((a.I + rpg1 - 1) / rpg1), ng2 = a.T * ((a.H + rpg2 - 1) / rpg2);
  const size_t fixed1 = i8 ? (size_t)a.T * ((size_t)a.H + (size_t)(a.H / 32) * 8)
                           : (size_t)a.T * a.fc1_chunks * kStagedWords * sizeof(uint32_t);
  const size_t fixed2 = i8 ? (size_t)a.T * a.k * ((size_t)a.I + (size_t)(a.I / 32) * 8)
                           : (size_t)a.T * a.k * a.fc2_chunks * kStagedWords * sizeof(uint32_t);
  const size_t l1 = fixed1 + (size_t)((ng1 + grid - 1) / grid) * rpg1 * 2 * sizeof(float);
  const size_t l2 = fixed2 + (size_t)((ng2 + grid - 1) / grid) * rpg2 * a.k * sizeof(float);
  return l1 > l2 ? l1 : l2;
}

constexpr size_t kMaxFusedLds = 150 * 1024;

template <int RI, int R, int ZK1, int ZK2, int INT8>
static bool launch_fused(const QmoeArgs& a, hipStream_t st) {
  auto kern = qmoe_fused_kernel<RI, R, ZK1, ZK2, INT8>;
  const int cus = a.num_cus > 0 ? a.num_cus : 256;
  // every work-group of the grid must be resident at once: the grid never exceeds the
  // occupancy of the kernel with the LDS it is launched with
  int per_cu = a.f_wpc;
  size_t lds = 0;
  for (; per_cu >= 1; --per_cu) {
    lds = fused_lds(a, R, (int64_t)cus * per_cu);
    if (lds == 0 || lds > kMaxFusedLds) return false;
    if (moe_resident_per_cu(kern, lds) >= per_cu) break;
  }
  if (per_cu < 1) return false;
  allow_lds(kern, lds);
  launch(kern, dim3((unsigned)(cus * per_cu)), dim3(kMoeStreamThreads), lds, st, a);
  return true;
}

template <int RI, int ZK>
static bool launch_fc1_dedupe(const QmoeArgs& a, hipStream_t st) {
  auto kern = qmoe_fc1_dedupe_kernel<RI, ZK>;
  if (a.mode != QMOE_FP || a.T < 2 || a.T > kDedupeMaxT || a.T * a.k > kMoeSortSlots) return false;
  const int64_t erows = 2 * a.I;
  if (erows * a.fc1_row_bytes >= (1LL << 31) || erows * a.fc1_nblk * 2 >= (1LL << 31)) return false;
  const int64_t rpg = (64 >> a.fc1_lpr_log2) * RI;
  // group count at its largest (every slot its own expert); the kernel deals the
  // actual groups, never more
  const int64_t ngroups = a.T * a.k * ((a.I + rpg - 1) / rpg);
  const size_t fixed = (size_t)a.T * a.fc1_chunks * kStagedWords * sizeof(uint32_t) + (size_t)kDedupeInts * sizeof(int);
  int64_t grid = 0;
  size_t lds = 0;
  if (!moe_stream_plan(kern, ngroups, fixed, (size_t)rpg * kDedupeMaxT * 2 * sizeof(float), a.num_cus, 1,
                       &grid, &lds))
    return false;
  allow_lds(kern, lds);
  launch(kern, dim3((unsigned)grid), dim3(kMoeStreamThreads), lds, st, a);
  return true;
}

bool qmoe_fused_plan(QmoeArgs& a, int candidate) {
  if (candidate < 0 || candidate >= kNumQmoeFused) return false;
  a.f_r2 = kQmoeFusedR2[candidate % 2];
  a.f_wpc = kQmoeFusedWpc[candidate / 2];
  // the limits launch_fused applies, at one work-group per compute unit (the most LDS
  // per work-group)
  const size_t lds = fused_lds(a, a.f_r2, a.num_cus > 0 ? a.num_cus : 256);
  return lds != 0 && lds <= kMaxFusedLds;
}

template <int INT8>
static bool launch_fused_zk(const QmoeArgs& a, hipStream_t st) {
  const bool z1 = a.fc1.zp != nullptr, z2 = a.fc2.zp != nullptr;
  if (a.f_r2 == 1)
    return z1 ? (z2 ? launch_fused<2, 1, 1, 1, INT8>(a, st) : launch_fused<2, 1, 1, 0, INT8>(a, st))
              : (z2 ? launch_fused<2, 1, 0, 1, INT8>(a, st) : launch_fused<2, 1, 0, 0, INT8>(a, st));
  return z1 ? (z2 ? launch_fused<2, 2, 1, 1, INT8>(a, st) : launch_fused<2, 2, 1, 0, INT8>(a, st))
            : (z2 ? launch_fused<2, 2, 0, 1, INT8>(a, st) : launch_fused<2, 2, 0, 0, INT8>(a, st));
}

hipError_t launch_qmoe_fused(const QmoeArgs& a, hipStream_t st) {
  const bool done = a.mode == QMOE_INT8_ACT ? launch_fused_zk<1>(a, st) : launch_fused_zk<0>(a, st);
  return done ? hipSuccess : hipErrorNotSupported;
}

hipError_t launch_qmoe_fc1(const QmoeArgs& a, int candidate, hipStream_t st) {
  const int rows_per_lane = candidate & 15;
  if (candidate & kQmoeDedupe) {
    bool done;
    if (rows_per_lane == 1) done = a.fc1.zp ? launch_fc1_dedupe<1, 1>(a, st) : launch_fc1_dedupe<1, 0>(a, st);
    else done = a.fc1.zp ? launch_fc1_dedupe<2, 1>(a, st) : launch_fc1_dedupe<2, 0>(a, st);
    if (done) return hipSuccess;
  }
  if (!(candidate & kQmoePerSlot)) {
    const bool zk = a.fc1.zp != nullptr;
    bool done;
    const int cap = (candidate & kQmoeOnePerCu) ? 1 : 1 << 20;
    if (a.mode == QMOE_INT8_ACT) {
      if (rows_per_lane == 1) done = zk ? launch_fc1_stream<1, 1, 1>(a, cap, st) : launch_fc1_stream<1, 0, 1>(a, cap, st);
      else done = zk ? launch_fc1_stream<2, 1, 1>(a, cap, st) : launch_fc1_stream<2, 0, 1>(a, cap, st);
    } else {
      if (rows_per_lane == 1) done = zk ? launch_fc1_stream<1, 1, 0>(a, cap, st) : launch_fc1_stream<1, 0, 0>(a, cap, st);
      else done = zk ? launch_fc1_stream<2, 1, 0>(a, cap, st) : launch_fc1_stream<2, 0, 0>(a, cap, st);
    }
    if (done) return hipSuccess;
  }
  const int subs = 64 >> a.fc1_lpr_log2;
  const int64_t rows_per_wg = 4LL * subs * rows_per_lane;
  const dim3 grid((unsigned)((a.I + rows_per_wg - 1) / rows_per_wg), (unsigned)(a.T * a.k));
  const size_t lds = qmoe_fc1_lds_bytes(a);
  if (a.mode == QMOE_INT8_ACT) {
    if (rows_per_lane == 1) launch((qmoe_fc1_kernel<1, 1>), grid, dim3(256), lds, st, a);
    else launch((qmoe_fc1_kernel<1, 2>), grid, dim3(256), lds, st, a);
  } else {
    allow_lds(qmoe_fc1_kernel<0, 1>, lds);
    allow_lds(qmoe_fc1_kernel<0, 2>, lds);
    if (rows_per_lane == 1) launch((qmoe_fc1_kernel<0, 1>), grid, dim3(256), lds, st, a);
    else launch((qmoe_fc1_kernel<0, 2>), grid, dim3(256), lds, st, a);
  }
  return hipSuccess;
}

hipError_t launch_qmoe_fc2(const QmoeArgs& a, int candidate, hipStream_t st) {
  const int rows_per_lane = candidate & 15;
  if (a.mode == QMOE_INT8_ACT) {
    // h -> int8 codes and scales once (into the scratch fc2 stages from)
    const int64_t groups = a.T * a.k * a.I / 32;
    const int64_t blocks = (groups + 7) / 8;
    launch(qmoe_quant_h_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.h, groups, a.hq_out,
                       a.hs_out);
  }
  if (!(candidate & kQmoePerSlot)) {
    const bool zk = a.fc2.zp != nullptr;
    bool done;
    const int cap = (candidate & kQmoeOnePerCu) ? 1 : 1 << 20;
    if (a.mode == QMOE_INT8_ACT) {
      if (rows_per_lane == 1) done = zk ? launch_fc2_stream<1, 1, 1>(a, cap, st) : launch_fc2_stream<1, 0, 1>(a, cap, st);
      else done = zk ? launch_fc2_stream<2, 1, 1>(a, cap, st) : launch_fc2_stream<2, 0, 1>(a, cap, st);
    } else {
      if (rows_per_lane == 1) done = zk ? launch_fc2_stream<1, 1, 0>(a, cap, st) : launch_fc2_stream<1, 0, 0>(a, cap, st);
      else done = zk ? launch_fc2_stream<2, 1, 0>(a, cap, st) : launch_fc2_stream<2, 0, 0>(a, cap, st);
    }
    if (done) return hipSuccess;
  }
  const int subs = 64 >> a.fc2_lpr_log2;
  const int64_t rows_per_wg = 4LL * subs * rows_per_lane;
  const dim3 grid((unsigned)((a.H + rows_per_wg - 1) / rows_per_wg), (unsigned)a.T);
  const size_t lds = qmoe_fc2_lds_bytes(a);
  if (a.mode == QMOE_INT8_ACT) {
    if (rows_per_lane == 1) launch((qmoe_fc2_kernel<1, 1>), grid, dim3(256), lds, st, a);
    else launch((qmoe_fc2_kernel<1, 2>), grid, dim3(256), lds, st, a);
  } else {
    allow_lds(qmoe_fc2_kernel<0, 1>, lds);
    allow_lds(qmoe_fc2_kernel<0, 2>, lds);
    if (rows_per_lane == 1) launch((qmoe_fc2_kernel<0, 1>), grid, dim3(256), lds, st, a);
    else launch((qmoe_fc2_kernel<0, 2>), grid, dim3(256), lds, st, a);
  }
  return hipSuccess;
}

}  // namespace qmm
