// Prefill (large M) path of MatMulNBits on the fp16 matrix cores
// ([P1] hip-ep PR 1318, "What", commit 1: the prefill tiles re-read A once per
// N block, so A is cast to fp16 once and fp32 C is written from the epilogue;
// "Performance"/Qwen study: prefill is compute bound).
//
// C[M][N] = A16 . W16^T (+ bias), with A16 = fp16(A) (cast once into the caller's
// workspace by launch_cast_pad_f16, rows padded with zeros to a multiple of 64) and
// W16 = fp16(fp32(fp32(q - zp) * s)), the round-to-nearest fp16 of the exact
// dequantized weight, built tile by tile in LDS.  Products are accumulated in fp32
// by v_mfma_f32_32x32x16_f16 in increasing k order (64 codes per stage), whatever
// the tile shape.
//
// Work-group: 512 threads (8 waves, two per SIMD so that one wave's matrix-core
// work overlaps the other's dequantization and LDS traffic), output tile
// BM x BN = 256 x 256, each wave a 64 x 128 part held as 2 x 4 MFMA blocks of
// 32 x 32 (fp32 accumulators).  Per 64-deep k stage, A[256][64] (fp16) comes into
// LDS by direct global->LDS loads and W16[256][64] is dequantized into LDS, both
// double buffered with one barrier per stage; the dequantization of the next stage
// is interleaved with the MFMA k steps of the current one.
//
// MFMA operand layout (32x32x16 f16): lane l holds row (or column) l % 32 and the 8
// consecutive k at 8 * (l / 32); accumulator v of lane l is row 8*(v/4) + 4*(l/32)
// + v%4, column l % 32.
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_skinny.h"

#include <algorithm>

namespace qmm {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NT = 512;      // threads
constexpr uint32_t kWord3 = 0x00020000u;  // raw buffer descriptor, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  const uint32_t n = bytes >= 0x7fffffff ? 0x7fffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, (int)kWord3);
}

// Weight data of one stage for one thread: 32 codes of W row n0 + t/2 (k half t%2)
// with the scale and zero point of each 16.
template <int BITS>
struct Stage {
  uint32_t w[BITS];  // 32 codes: BITS dwords (2-bit -> 2, 3-bit -> 3, 4-bit -> 4, 8-bit -> 8)
  _Float16 sc[2];    // affine scale
  _Float16 zh[2];
  uint32_t zb[2];
  float am[2];       // codebook absmax
};

template <int CT>
__device__ __forceinline__ void store_c(void* C, int64_t i, float v) {
  if constexpr (CT == QMM_F32) ((float*)C)[i] = v;
  else if constexpr (CT == QMM_F16) ((uint16_t*)C)[i] = f32_to_f16(v);
  else ((uint16_t*)C)[i] = f32_to_bf16(v);
}

template <int CT>
__device__ __forceinline__ float load_bias(const void* b, int64_t i) {
  if constexpr (CT == QMM_F32) return ((const float*)b)[i];
  else if constexpr (CT == QMM_F16) return f16_to_f32(((const uint16_t*)b)[i]);
  else return bf16_to_f32(((const uint16_t*)b)[i]);
}

// LDS tiles: 256 rows of 64 fp16 (128 bytes, no padding); the 16-byte piece p of row
// r sits at piece position p ^ ((r / 2) % 8).  The LDS serves 16 lanes (256 bytes) of a
// 16-byte access per cycle, and a 256-byte line holds two rows: the 16 consecutive rows
// that 16 lanes read at one k then fall on 16 different 16-byte bank groups (with the
// position p ^ (r % 8), rows r and r + 8 met in one bank group on every operand read
// and every dequantized-weight store: 43% of the LDS cycles were conflict stalls on
// MI355X).  A is double buffered and filled by
// direct global->LDS loads (no registers on the way); W16 is double buffered and
// written by the dequantization.
__shared__ __attribute__((aligned(16))) uint8_t pf_a0[BM * 128];
__shared__ __attribute__((aligned(16))) uint8_t pf_a1[BM * 128];
__shared__ __attribute__((aligned(16))) uint8_t pf_b0[BN * 128];
__shared__ __attribute__((aligned(16))) uint8_t pf_b1[BN * 128];
__shared__ float pf_cb[16];  // codebook (16 entries, one per bank)

__device__ __forceinline__ uint32_t swz(int row, int piece) {
  return (uint32_t)row * 128u + (uint32_t)((piece ^ ((row >> 1) & 7)) << 4);
}

// FMT: GEMV_AFFINE (w = (q - zp) * s) or GEMV_CODEBOOK (BITS = 4, w = codebook[q] * absmax).
template <int FMT, int BITS, int ZK, int CT>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillArgs p) {
  if constexpr (FMT == GEMV_CODEBOOK) {
    if (threadIdx.x < 16) pf_cb[threadIdx.x] = p.codebook[threadIdx.x];
  }
  // tile order (work-groups are dealt round-robin over the 8 XCDs)
  // blockIdx.x = ks * tiles_grid + tile index; split ks covers stages
  // [ks * spl, min((ks + 1) * spl, nsteps)) of the reduction
  const int ks = (int)blockIdx.x / p.tiles_grid;
  const int i = (int)blockIdx.x - ks * p.tiles_grid;
  const int x = i & 7, j = i >> 3;
  int nt, mt;
  if (p.mtiles == 8) {
    // one M tile per XCD: its A rows (256 x K fp16) stay in that XCD's L2 while the
    // XCD walks every N tile; the packed weights are shared through the last-level cache
    mt = x;
    nt = j;
  } else {
    // the M tiles of one N tile on one XCD: the packed weights of that N tile are
    // read into one L2
    nt = (j / p.mtiles) * 8 + x;
    mt = j % p.mtiles;
  }
  if (nt >= p.ntiles) return;
  const int m0 = mt * BM, n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 waves, 64 x 128 each
  const int Kp = (int)p.Kp;
  const int nsteps = Kp / BK;
  const int s_begin = ks * p.spl;
  const int nlocal = (s_begin + p.spl < nsteps ? s_begin + p.spl : nsteps) - s_begin;
  const int nblk = (int)p.nblk;
  const int blog = p.block_log2;

  // A rows of this thread's direct loads: wave w fills rows 32w .. 32w + 31 with four
  // 8-row loads; lane l takes row 32w + 8i + l/8 at piece position l % 8, i.e. global
  // piece (l % 8) ^ ((row / 2) % 8).  Rows past M read row M - 1 (results unused).
  const uint8_t* a_src[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = wave * 32 + q * 8 + (lane >> 3);
    int grow = m0 + row;
    grow = grow < (int)p.M ? grow : (int)p.M - 1;
    const int piece = (lane & 7) ^ ((row >> 1) & 7);
    a_src[q] = (const uint8_t*)p.A16 + ((int64_t)grow * p.lda) * 2 + piece * 16;
  }
  // plain global addresses (no range check): the stage index is clamped to the last
  // stage, so no load ever leaves the A16 rows
  auto load_a = [&](int s, uint8_t* dst) {
    const int sc = s < nsteps ? s : nsteps - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[q] + (int64_t)sc * (BK * 2)),
                                       (__attribute__((address_space(3))) void*)(dst + (wave * 32 + q * 8) * 128),
                                       16, 0, 0);
  };

  // this thread's W row n0 + tid/2, k half tid%2 (32 codes per stage)
  const int r2 = tid >> 1, h = tid & 1;
  const __amdgpu_buffer_rsrc_t rW = rsrc(p.W, p.N * p.row_bytes);
  const __amdgpu_buffer_rsrc_t rS = FMT == GEMV_CODEBOOK ? rsrc(p.absmax, p.N * p.nblk * 4)
                                                          : rsrc(p.scales, p.N * p.nblk * 2);
  __amdgpu_buffer_rsrc_t rZ = rS;
  if constexpr (ZK == 1) rZ = rsrc(p.zp, p.N * p.zp_row_bytes);
  if constexpr (ZK == 2) rZ = rsrc(p.zp, p.N * p.nblk * 2);
  const int wrow = n0 + r2;
  const uint32_t w_off = (uint32_t)((int64_t)wrow * p.row_bytes) + (uint32_t)h * (32 * BITS / 8);
  const uint32_t s_off = (uint32_t)((int64_t)wrow * nblk * 2);
  const uint32_t z_off = (uint32_t)((int64_t)wrow * p.zp_row_bytes);
  const int kmax_blk = nblk - 1;

  auto load_w = [&](int s, Stage<BITS>& st) {
    const int k0 = s * BK;
    const uint32_t wo = w_off + (uint32_t)(k0 * BITS / 8);
#pragma unroll
    for (int d = 0; d < BITS; ++d) st.w[d] = __builtin_amdgcn_raw_buffer_load_b32(rW, (int)(wo + 4u * d), 0, 0);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      int blk = (k0 + 32 * h + 16 * g) >> blog;
      blk = blk < kmax_blk ? blk : kmax_blk;  // codes past the row end meet zero A
      if constexpr (FMT == GEMV_CODEBOOK) {
        st.am[g] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, (int)(2u * s_off + 4u * blk), 0, 0));
        continue;
      }
      st.sc[g] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rS, (int)(s_off + 2u * blk), 0, 0));
      if constexpr (ZK == 1) {
        const int bit = blk * BITS;
        const uint32_t zo = z_off + (uint32_t)(bit >> 3);
        uint32_t zb = __builtin_amdgcn_raw_buffer_load_b8(rZ, (int)zo, 0, 0);
        // a 3-bit field may continue into the next byte (past the buffer it reads 0)
        if constexpr (BITS == 3) zb |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rZ, (int)(zo + 1u), 0, 0) << 8;
        st.zb[g] = BITS == 8 ? zb : zb >> (bit & 7);
      } else if constexpr (ZK == 2) {
        st.zh[g] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rZ, (int)(s_off + 2u * blk), 0, 0));
      }
    }
  };

  // dequantize part q (codes 8q .. 8q+7) of this thread's 32 codes into row r2 of dst
  auto store_part = [&](const Stage<BITS>& st, uint8_t* dst, int q) {
    const int g = q >> 1;
    if constexpr (FMT == GEMV_CODEBOOK) {
      // w = fp32(codebook[q] * absmax), then fp16 (round to nearest even)
      const uint32_t xw = st.w[q];  // 8 codes
      const float am = st.am[g];
      uint32_t o[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x2 w;
        w.x = __fmul_rn(pf_cb[(xw >> (8 * jj)) & 15u], am);
        w.y = __fmul_rn(pf_cb[(xw >> (8 * jj + 4)) & 15u], am);
        o[jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2));
      }
      *(uint4*)(dst + swz(r2, 4 * h + q)) = make_uint4(o[0], o[1], o[2], o[3]);
      return;
    }
    const float sc = (float)st.sc[g];
    float z;
    if constexpr (ZK == 1) z = BITS == 8 ? (float)(int8_t)st.zb[g] : (float)(st.zb[g] & ((1u << BITS) - 1u));
    else if constexpr (ZK == 2) z = (float)st.zh[g];
    else z = p.zconst;
    // codes as exact fp32 integers, two per conversion: 2-bit codes masked into e2m1
    // nibbles are q/2 (scaled by 2), 4-bit codes masked into e4m3 bytes are q * 2^-9
    // (scaled by 2^9); 3-bit and signed 8-bit codes are extracted one by one
    float qv[8];
    if constexpr (BITS == 3) {
      // codes 8q .. 8q+7: the 24-bit field at bit 24 q of this thread's 96 bits
      const uint32_t xw = q == 0 ? st.w[0] : q == 1 ? __builtin_amdgcn_alignbit(st.w[1], st.w[0], 24)
                        : q == 2 ? __builtin_amdgcn_alignbit(st.w[2], st.w[1], 16) : (st.w[2] >> 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = (float)__builtin_amdgcn_ubfe(xw, 3 * i, 3);
    } else if constexpr (BITS == 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[i] = (float)(int)__builtin_amdgcn_sbfe((int)st.w[2 * q], 8 * i, 8);
        qv[4 + i] = (float)(int)__builtin_amdgcn_sbfe((int)st.w[2 * q + 1], 8 * i, 8);
      }
    } else if constexpr (BITS == 2) {
      const uint32_t xw = st.w[q >> 1] >> (16 * (q & 1));  // 8 codes in the low 16 bits
      const uint32_t ev = xw & 0x3333u, od = (xw >> 2) & 0x3333u;
      const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 2.0f, 0);
      const f32x2 o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 2.0f, 0);
      const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 2.0f, 1);
      const f32x2 o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 2.0f, 1);
      qv[0] = e0.x; qv[2] = e0.y; qv[1] = o0.x; qv[3] = o0.y;
      qv[4] = e1.x; qv[6] = e1.y; qv[5] = o1.x; qv[7] = o1.y;
    } else {
      const uint32_t xw = st.w[q];  // 8 codes
      const uint32_t lo = xw & 0x0F0F0F0Fu, hi = (xw >> 4) & 0x0F0F0F0Fu;
      const f32x2 l0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, false);
      const f32x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, false);
      const f32x2 l1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, true);
      const f32x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, true);
      qv[0] = l0.x; qv[2] = l0.y; qv[4] = l1.x; qv[6] = l1.y;
      qv[1] = h0.x; qv[3] = h0.y; qv[5] = h1.x; qv[7] = h1.y;
    }
    uint32_t o[4];
    if (ZK == 1 || (ZK == 0 && p.zconst_fma)) {
      // q - z is exact for every code and z * s is exact (packed integer zero points, or
      // a constant that passed zconst_fma_exact), so one fma gives fp32((q - z) * s)
      const float nzs = -(z * sc);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x2 w;
        w.x = __fmaf_rn(qv[2 * jj], sc, nzs);
        w.y = __fmaf_rn(qv[2 * jj + 1], sc, nzs);
        o[jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2));  // round to nearest even
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x2 w;
        w.x = __fmul_rn(__fsub_rn(qv[2 * jj], z), sc);
        w.y = __fmul_rn(__fsub_rn(qv[2 * jj + 1], z), sc);
        o[jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2));  // round to nearest even
      }
    }
    *(uint4*)(dst + swz(r2, 4 * h + q)) = make_uint4(o[0], o[1], o[2], o[3]);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  // operand rows of this lane: A rows wm*64 + 32a + lane%32, W rows wn*128 + 32b + lane%32;
  // all have (row / 2) % 8 == (lane / 2) % 8
  const uint32_t a_row0 = (uint32_t)(wm * 64 + (lane & 31)) * 128u;
  const uint32_t b_row0 = (uint32_t)(wn * 128 + (lane & 31)) * 128u;
  const int hi = lane >> 5, l7 = (lane >> 1) & 7;  // (row / 2) % 8 of the lane's operand rows

  // matrix-core work of one stage (tiles ab, bb); after each 16-deep k step, one part
  // of the next stage's weights (st) is dequantized into sdst
  auto compute = [&](const uint8_t* ab, const uint8_t* bb, const Stage<BITS>& st, uint8_t* sdst,
                     bool do_store) {
    f16x8 af[2][2], bf[2][4];
    auto frags = [&](int q, f16x8 (&fa)[2], f16x8 (&fb)[4]) {
      const uint32_t pos = (uint32_t)(((2 * q + hi) ^ l7) << 4);
#pragma unroll
      for (int a = 0; a < 2; ++a) fa[a] = *(const f16x8*)(ab + a_row0 + a * 32 * 128 + pos);
#pragma unroll
      for (int b = 0; b < 4; ++b) fb[b] = *(const f16x8*)(bb + b_row0 + b * 32 * 128 + pos);
    };
    frags(0, af[0], bf[0]);
#pragma unroll
    for (int q = 0; q < BK / 16; ++q) {
      if (q + 1 < BK / 16) frags(q + 1, af[(q + 1) & 1], bf[(q + 1) & 1]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[q & 1][a], bf[q & 1][b], acc[a][b], 0, 0, 0);
      if (do_store) store_part(st, sdst, q);
    }
  };

  // stage s computes from (pf_a[s%2], pf_b[s%2]); during it, A of stage s + 1 is
  // loaded into pf_a[(s+1)%2], the weights of stage s + 2 into register set s%2, and
  // the weights of stage s + 1 (register set (s+1)%2) are dequantized into
  // pf_b[(s+1)%2].  Every load issued in a stage is waited for at its closing barrier.
  Stage<BITS> w0, w1;
  // stage indices below are local to the split: global stage = s_begin + local
  load_a(s_begin, pf_a0);
  load_w(s_begin, w0);
  load_w(s_begin + 1, w1);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) store_part(w0, pf_b0, q);
  __syncthreads();
  int s = 0;
  for (; s + 2 <= nlocal; s += 2) {
    load_a(s_begin + s + 1, pf_a1);
    load_w(s_begin + s + 2, w0);
    compute(pf_a0, pf_b0, w1, pf_b1, true);
    __syncthreads();
    if (s + 2 < nlocal) load_a(s_begin + s + 2, pf_a0);
    load_w(s_begin + s + 3, w1);
    compute(pf_a1, pf_b1, w0, pf_b0, s + 2 < nlocal);
    __syncthreads();
  }
  if (s < nlocal) compute(pf_a0, pf_b0, w1, pf_b1, false);  // odd number of stages

  if (p.splits > 1) {
    // split reduction: fp32 partial sums of this split, summed in split order (and the
    // bias added) by reduce_splits_kernel
    float* P = p.partials + (int64_t)ks * p.M * p.ldc;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int col = n0 + wn * 128 + b * 32 + (lane & 31);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * 64 + a * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (col < p.N && row < p.M) P[(int64_t)row * p.ldc + col] = acc[a][b][v];
        }
    }
    return;
  }
  // epilogue: x row scale of the activation cast, + bias, convert, store (rows and
  // columns past the end are skipped)
  float rsv[2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + wm * 64 + a * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      rsv[a][v] = (p.row_scale && row < p.M) ? p.row_scale[row] : 1.0f;
    }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int col = n0 + wn * 128 + b * 32 + (lane & 31);
    const bool col_ok = col < p.N;
    const float bv = (p.bias && col_ok) ? load_bias<CT>(p.bias, col) : 0.0f;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 64 + a * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (col_ok && row < p.M) store_c<CT>(p.C, (int64_t)row * p.ldc + col, acc[a][b][v] * rsv[a][v] + bv);
      }
    }
  }
}

// C[m][n] = (((P[0] + P[1]) + ...) + P[S-1])[m][n] * rs[m] + bias[n], in the type of C
// (rs = the activation cast's row scales, or 1 when NULL).
template <int CT>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* P, int S, int64_t M, int64_t N,
                                                            int64_t ldc, const float* rs, const void* bias, void* C) {
  const int64_t total = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / N, n = i - m * N;
    float v = P[m * ldc + n];
    for (int k = 1; k < S; ++k) v += P[(int64_t)k * M * ldc + m * ldc + n];
    if (rs) v *= rs[m];
    if (bias) v += load_bias<CT>(bias, n);
    store_c<CT>(C, m * ldc + n, v);
  }
}

template <int FMT, int BITS, int ZK, int CT>
void launch_one(const PrefillArgs& p, dim3 grid, hipStream_t st) {
  launch((prefill_kernel<FMT, BITS, ZK, CT>), grid, dim3(NT), 0, st, p);
}

template <int FMT, int BITS, int ZK>
void launch_ct(const PrefillArgs& p, dim3 grid, hipStream_t st) {
  if (p.c_type == QMM_F32) launch_one<FMT, BITS, ZK, QMM_F32>(p, grid, st);
  else if (p.c_type == QMM_F16) launch_one<FMT, BITS, ZK, QMM_F16>(p, grid, st);
  else launch_one<FMT, BITS, ZK, QMM_BF16>(p, grid, st);
}

}  // namespace

hipError_t launch_reduce_splits(const float* P, int S, int64_t M, int64_t N, int64_t ldc, const float* rs,
                                const void* bias, void* C, int c_type, hipStream_t st) {
  int64_t blocks = (M * N + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (c_type == QMM_F32)
    launch(reduce_splits_kernel<QMM_F32>, dim3((unsigned)blocks), dim3(256), 0, st, P, S, M, N, ldc, rs, bias, C);
  else if (c_type == QMM_F16)
    launch(reduce_splits_kernel<QMM_F16>, dim3((unsigned)blocks), dim3(256), 0, st, P, S, M, N, ldc, rs, bias, C);
  else
    launch(reduce_splits_kernel<QMM_BF16>, dim3((unsigned)blocks), dim3(256), 0, st, P, S, M, N, ldc, rs, bias, C);
  return hipSuccess;
}

int prefill_splits(int64_t M, int64_t N, int64_t Kp) {
  // Splits of the reduction when the 256 x 256 output tiles do not fill the chip.
  // Cost in stage times (one 256 x 256 x 64 tile step, about 2.5 us): rounds of work
  // groups over 256 slots (one 512-thread group per compute unit) times stages per
  // split, plus the fp32 partial sums written and read back (8 bytes per output per
  // split at about 4 TB/s) and one more launch.  The smallest split count of least
  // cost wins (at most 64, at most one per stage).  A function of the shape only, so
  // the summation order never depends on the device.
  constexpr int64_t kSlots = 256;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t nsteps = Kp / BK;
  if (tiles >= kSlots) return 1;
  int best = 1;
  double best_cost = (double)((tiles + kSlots - 1) / kSlots) * (double)nsteps;
  for (int s = 2; s <= 64 && s <= nsteps; ++s) {
    const double cost = (double)((tiles * s + kSlots - 1) / kSlots) * (double)((nsteps + s - 1) / s) +
                        (double)s * (double)M * (double)N * 8.0 / 1e7 + 1.0;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

hipError_t launch_prefill(PrefillArgs p, hipStream_t st) {
  // buffer offsets are 32-bit: split M and N so that every operand slice stays
  // below 2^31 bytes (one launch per slice)
  const int64_t lim = (int64_t)1 << 30;
  int64_t mstep = std::max<int64_t>(BM, (lim / (p.Kp * 2)) / BM * BM);
  int64_t nstep = std::max<int64_t>(BN, (lim / std::max<int64_t>(p.row_bytes, p.nblk * 4)) / BN * BN);
  const int zk = p.zp_kind == QMM_ZP_PACKED ? 1 : p.zp_kind == QMM_ZP_F16 ? 2 : 0;
  const size_t c_es = p.c_type == QMM_F32 ? 4 : 2;
  const bool sliced = mstep < p.M || nstep < p.N;
  for (int64_t m0 = 0; m0 < p.M; m0 += mstep) {
    for (int64_t n0 = 0; n0 < p.N; n0 += nstep) {
      PrefillArgs q = p;
      q.M = std::min(mstep, p.M - m0);
      q.N = std::min(nstep, p.N - n0);
      q.A16 = p.A16 + m0 * p.lda;
      if (p.row_scale) q.row_scale = p.row_scale + m0;
      q.W = p.W + n0 * p.row_bytes;
      if (p.scales) q.scales = p.scales + n0 * p.nblk;
      if (p.absmax) q.absmax = p.absmax + n0 * p.nblk;
      if (zk == 1) q.zp = (const uint8_t*)p.zp + n0 * p.zp_row_bytes;
      if (zk == 2) q.zp = (const uint16_t*)p.zp + n0 * p.nblk;
      if (p.bias) q.bias = (const uint8_t*)p.bias + n0 * (int64_t)c_es;
      q.C = (uint8_t*)p.C + (m0 * p.ldc + n0) * (int64_t)c_es;
      q.ntiles = (int)((q.N + BN - 1) / BN);
      q.mtiles = (int)((q.M + BM - 1) / BM);
      const int64_t groups = (q.ntiles + 7) / 8;
      q.tiles_grid = (int)(groups * 8 * q.mtiles);
      q.splits = prefill_splits(q.M, q.N, q.Kp);
      q.spl = (int)((q.Kp / BK + q.splits - 1) / q.splits);
      if (q.splits > 1 && (!p.partials || sliced)) q.splits = 1, q.spl = (int)(q.Kp / BK);
      const dim3 grid((unsigned)(q.tiles_grid * q.splits));
      if (q.fmt == GEMV_CODEBOOK) {
        launch_ct<GEMV_CODEBOOK, 4, 0>(q, grid, st);
      } else if (q.bits == 2) {
        if (zk == 1) launch_ct<GEMV_AFFINE, 2, 1>(q, grid, st);
        else if (zk == 2) launch_ct<GEMV_AFFINE, 2, 2>(q, grid, st);
        else launch_ct<GEMV_AFFINE, 2, 0>(q, grid, st);
      } else if (q.bits == 3) {
        if (zk == 1) launch_ct<GEMV_AFFINE, 3, 1>(q, grid, st);
        else if (zk == 2) launch_ct<GEMV_AFFINE, 3, 2>(q, grid, st);
        else launch_ct<GEMV_AFFINE, 3, 0>(q, grid, st);
      } else if (q.bits == 8) {
        if (zk == 1) launch_ct<GEMV_AFFINE, 8, 1>(q, grid, st);
        else if (zk == 2) launch_ct<GEMV_AFFINE, 8, 2>(q, grid, st);
        else launch_ct<GEMV_AFFINE, 8, 0>(q, grid, st);
      } else {
        if (zk == 1) launch_ct<GEMV_AFFINE, 4, 1>(q, grid, st);
        else if (zk == 2) launch_ct<GEMV_AFFINE, 4, 2>(q, grid, st);
        else launch_ct<GEMV_AFFINE, 4, 0>(q, grid, st);
      }
      if (q.splits > 1) launch_reduce_splits(q.partials, q.splits, q.M, q.N, q.ldc, q.row_scale, q.bias, q.C, q.c_type, st);
    }
  }
  return hipSuccess;
}

}  // namespace qmm
