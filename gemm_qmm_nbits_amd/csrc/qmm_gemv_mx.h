// Matrix-core form of the 2-bit integer-plane GEMV at M = 1 ([P1] hip-ep PR 1318,
// "What": the decode GEMV over 2-bit affine weights; the fixed-point planes of A are
// those of qmm_gemv_ip.h).  It computes the same per-chunk integer sums
// S_p = sum_k digit_p(a_int[k]) q[k] as the v_dot8 kernel, on the matrix cores, and then
// runs the same fp32 steps in the same order, so its results equal that kernel's bit
// for bit:
//   * v_mfma_scale_f32_16x16x128_f8f6f4 with A in e4m3 and B in e2m1: a 2-bit code
//     masked into an e2m1 nibble is q / 2 exactly and the B scale 2^1 restores q; every
//     4-bit digit (the signed top one included) is exact in e4m3; every product and
//     every sum (at most 64 * 15 * 3) is an exact integer in fp32;
//   * B columns are 16 weight rows; a pair of steps covers four 64-code chunks, lane
//     group g loading chunk g (16 bytes) and the two steps taking its two halves;
//   * two accumulations per pair, each over two chunks: A operand rows 8c + 4h + v
//     carry digit plane 3h + v of chunk c (k < 64) and of chunk 2 + c (k >= 64) of
//     the pair, and the first accumulation's B keeps only the k < 64 lane groups, the
//     second's only the others, so lane group 2c + h of the result holds, per column,
//     the three sums of one half (lo = planes 0..2, hi = planes 3..5) of one chunk;
//   * lo + 16 S + 256 S' is exact, a row swap pairs lo with hi, and
//     P = fma(hi, 4096, lo), the outlier term, the zero-point fold and the scale follow
//     as in the v_dot8 kernel;
//   * chunk j of a row goes to partial j mod LPR in increasing order, and the partials
//     meet in the v_dot8 kernel's xor-butterfly tree (level 1 across the two chunk
//     parities, the rest across a lane's slots).
// A is staged once per work-group in the operand layout (4 KiB per 256 codes), so the
// form serves rows whose operand fits in LDS (K up to about 9000 codes).
#pragma once
#include "qmm_gemv_ip.h"

namespace qmm {

typedef int mx_i32x8 __attribute__((ext_vector_type(8)));
typedef float mx_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMxThreads = 1024;  // 16 waves share one staged operand
constexpr int kMxDepth = 4;       // ring of pair buffers: depth - 1 pairs in flight

template <int R>
struct MxBuf {
  uint4 w[R];           // chunk 4u + lane group of each row (16 bytes)
  _Float16 zh[R][2];    // fp16 zero points of the lane's two chunks
  uint32_t z[R][2];     // packed zero-point bytes
  uint32_t zsh[R][2];   // bit offsets of the codes in them
};

// Stage chunks [0, SC) of the single A row in the operand layout (SC a multiple of 4).
template <int AT, typename Issued>
__device__ __forceinline__ void stage_planes_mx(const GemvArgs& g, uint32_t* aop, f32x4* meta, uint32_t* trash,
                                                int SC, Issued&& issued) {
  if (g.a_vec)
    stage_planes_impl<2, AT, 64, 1, true, true, true>(g, aop, meta, trash, 0, SC, issued);
  else
    stage_planes_impl<2, AT, 64, 1, false, true, true>(g, aop, meta, trash, 0, SC, issued);
}

// T2 = pairs of steps (256 codes, four chunks) per row, a multiple of LPRH / 2 (LPRH =
// half the lanes per row of the v_dot8 kernel).  Lane group g of a wave loads chunk
// 4u + g of its 16 rows for pair u; the two steps of the pair take its halves, and the
// pair's two accumulations hold chunks 4u, 4u + 1 (rows 0..7 / 8..15 of the first) and
// 4u + 2, 4u + 3 (the second).  The epilogue of lane group g handles chunks
// 4u + g / 2 and 4u + 2 + g / 2: slot 2 (u mod LPRH / 2) + d of the lane is partial
// 2 slot + g / 2 of the v_dot8 kernel.  Scales (block 64: one per chunk) are loaded
// once per round of LPRH / 2 pairs, 16 bytes per lane, and paired between lane groups.
template <int AT, int R, int LPRH, int ZK>
__global__ __launch_bounds__(kMxThreads) void gemv_mx_kernel(GemvArgs g, int T2) {
  constexpr int NW = kMxThreads / 64;
  constexpr int D = kMxDepth;
  constexpr int PR = LPRH / 2;   // pairs per round
  constexpr int NSQ = LPRH / 8;  // 16-byte scale loads per lane per round
  static_assert(PR % D == 0 && PR >= D, "the ring depth divides a round");
  extern __shared__ float lds[];
  const int SC = 4 * T2;
  uint32_t* aop = (uint32_t*)lds;            // T2 pairs x 1024 words
  f32x4* meta = (f32x4*)(aop + T2 * 1024);   // one record per chunk
  uint32_t* trash = (uint32_t*)(meta + SC);  // 16 words nothing reads
  float* out_lds = (float*)(trash + 16);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;  // lane group: the chunk it loads, the k quarter of B
  const int col = lane & 15;
  const int sig = lg >> 1;   // parity of the chunks whose epilogue this lane runs
  const uint32_t ssh = 16u * (uint32_t)sig;
  constexpr uint32_t kM = 0x33333333u;
  const uint32_t m1 = lg < 2 ? kM : 0u;  // B of the first accumulation: chunks 4u, 4u + 1
  const uint32_t m2 = lg < 2 ? 0u : kM;  // of the second: chunks 4u + 2, 4u + 3
  const int rpg = 16 * R;
  const int N = (int)g.N;
  const int ngroups = (N + rpg - 1) / rpg;
  const int groups_lo = ngroups / gridDim.x, extra = ngroups % gridDim.x;
  const int g_begin = blockIdx.x * groups_lo + (blockIdx.x < extra ? blockIdx.x : extra);
  const int g_end = g_begin + groups_lo + (blockIdx.x < extra ? 1 : 0);
  if (g_begin >= g_end) return;
  const int wave_groups = g_end - g_begin > wave ? (g_end - g_begin - wave + NW - 1) / NW : 0;
  const int nblk = (int)g.nblk;  // a multiple of 8: every chunk of a pair lies in the row
  const uint32_t row_bytes = (uint32_t)g.row_bytes;
  const float zconst = g.zp_kind == QMM_ZP_UNIFORM ? g.uniform_zp : 2.0f;
  const uint32_t zrow_bytes = (uint32_t)g.zp_row_bytes;

  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W, (uint32_t)(g.N * g.row_bytes));
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(g.scales, (uint32_t)(g.N * g.nblk * 2));
  __amdgpu_buffer_rsrc_t rZ = rS;
  if constexpr (ZK == 1) rZ = make_rsrc(g.zp, (uint32_t)(g.N * g.zp_row_bytes));
  if constexpr (ZK == 2) rZ = make_rsrc(g.zp, (uint32_t)(g.N * g.nblk * 2));

  // fetch cursor: per-row byte offsets of pair 0 of the current group, and the pair
  uint32_t fw[R], fs[R], fz[R];
  int fit = 0, fgrp = g_begin + wave;
  auto set_rows = [&](int grp) {
    // past the wave's own groups the cursor moves to rows past N: those loads read
    // past every buffer's range, return 0 and move no data
    const int gq = grp < g_end ? grp : ngroups;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = (uint32_t)(gq * rpg + 16 * r + col);
      fw[r] = row * row_bytes + 16u * (uint32_t)lg;
      fs[r] = row * (uint32_t)nblk * 2u + 16u * (uint32_t)(lg & 1);
      if constexpr (ZK == 1) fz[r] = row * zrow_bytes;
      if constexpr (ZK == 2) fz[r] = row * (uint32_t)nblk * 2u;
    }
  };
  set_rows(fgrp);
  // scales of the round that starts at the cursor: lane groups 0 / 2 take chunks
  // 16q + 0..7 of it, 1 / 3 chunks 16q + 8..15
  auto fetch_scales = [&](uint4 (&raw)[R][NSQ]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int q = 0; q < NSQ; ++q) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rS, (int)(fs[r] + (uint32_t)(fit * 8 + 32 * q)), 0, 0);
        raw[r][q] = make_uint4(v[0], v[1], v[2], v[3]);
      }
  };
  auto fetch = [&](MxBuf<R>& b) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)(fw[r] + (uint32_t)(fit * 64)), 0, 0);
      b.w[r] = make_uint4(v[0], v[1], v[2], v[3]);
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t ch = (uint32_t)(4 * fit + 2 * d + sig);
        if constexpr (ZK == 1) {
          const uint32_t bit = ch * 2u;
          b.z[r][d] = __builtin_amdgcn_raw_buffer_load_b8(rZ, (int)(fz[r] + (bit >> 3)), 0, 0);
          b.zsh[r][d] = bit & 7u;
        } else if constexpr (ZK == 2) {
          b.zh[r][d] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rZ, (int)(fz[r] + ch * 2u), 0, 0));
        }
      }
    }
    if (++fit == T2) {
      fit = 0;
      fgrp += NW;
      set_rows(fgrp);
    }
  };

  // operand slots the staging leaves alone (rows 4h + 3, and the lane groups of the
  // other chunk of a pair half) hold zeros
  for (int i = threadIdx.x; i < T2 * 256; i += kMxThreads) {
    const int la = i & 63, r = la & 15;
    if ((r & 3) == 3 || (la >> 5) != (r >> 3)) ((uint4*)aop)[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  MxBuf<R> buf[D];
  uint4 sraw[R][NSQ];
  stage_planes_mx<AT>(g, aop, meta, trash, SC, [&] {
    fetch_scales(sraw);
#pragma unroll
    for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
  });
  __syncthreads();

  float acc[R][LPRH];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < LPRH; ++s) acc[r][s] = 0.0f;
  uint32_t sc[R][NSQ][8];  // the round's scales: dword k of set q holds chunks 16q + 2k, + 1

  int cit = 0, cgrp = g_begin + wave;
  const int total = wave_groups * T2;
  const mx_f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  auto pair = [&](MxBuf<R>& cb, MxBuf<R>& nx, int i) {
    if (i == 0) {
      // the round's scales: lane groups 2k and 2k + 1 exchange their halves
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < NSQ; ++q) {
          const uint32_t v[4] = {sraw[r][q].x, sraw[r][q].y, sraw[r][q].z, sraw[r][q].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const auto sw = __builtin_amdgcn_permlane16_swap(v[k], v[k], false, false);
            sc[r][q][k] = sw[0];
            sc[r][q][4 + k] = sw[1];
          }
        }
    }
    if (i == PR - (D - 1)) fetch_scales(sraw);  // the fetch below starts the next round
    fetch(nx);
    const uint4* ap = (const uint4*)(aop + cit * 1024);
    const uint4 xa = ap[lane], xb = ap[64 + lane], ya = ap[128 + lane], yb = ap[192 + lane];
    // one operand per step: chunks 4u, 4u + 1 in the low half (k < 64), 4u + 2, 4u + 3 in
    // the high half; B keeps one half per accumulation (the other lane groups zero)
    const mx_i32x8 Aa = {(int)xa.x, (int)xa.y, (int)xa.z, (int)xa.w, (int)ya.x, (int)ya.y, (int)ya.z, (int)ya.w};
    const mx_i32x8 Ab = {(int)xb.x, (int)xb.y, (int)xb.z, (int)xb.w, (int)yb.x, (int)yb.y, (int)yb.z, (int)yb.w};
    f32x4 mt[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) mt[d] = meta[4 * cit + 2 * d + sig];
    const bool any_out = __builtin_amdgcn_ballot_w64(mt[0].z != 0.0f || mt[1].z != 0.0f) != 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint4 x = cb.w[r];
      const uint32_t e0 = x.x >> 2, e1 = x.y >> 2, e2 = x.z >> 2, e3 = x.w >> 2;
      const mx_i32x8 B1a = {(int)(x.x & m1), (int)(e0 & m1), (int)(x.y & m1), (int)(e1 & m1), 0, 0, 0, 0};
      const mx_i32x8 B1b = {(int)(x.z & m1), (int)(e2 & m1), (int)(x.w & m1), (int)(e3 & m1), 0, 0, 0, 0};
      const mx_i32x8 B2a = {(int)(x.x & m2), (int)(e0 & m2), (int)(x.y & m2), (int)(e1 & m2), 0, 0, 0, 0};
      const mx_i32x8 B2b = {(int)(x.z & m2), (int)(e2 & m2), (int)(x.w & m2), (int)(e3 & m2), 0, 0, 0, 0};
      // A e4m3 (cbsz 0), B e2m1 (blgp 4); scales 2^0 and 2^1
      mx_f32x4 acc2[2];
      acc2[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aa, B1a, zero4, 0, 4, 0, 0x7f7f7f7f, 0, (int)0x80808080);
      acc2[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aa, B2a, zero4, 0, 4, 0, 0x7f7f7f7f, 0, (int)0x80808080);
      acc2[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Ab, B1b, acc2[0], 0, 4, 0, 0x7f7f7f7f, 0, (int)0x80808080);
      acc2[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Ab, B2b, acc2[1], 0, 4, 0, 0x7f7f7f7f, 0, (int)0x80808080);
      float P[2], scv[2], z[2];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int slot = 2 * (i % PR) + d;
        const mx_f32x4 dd = acc2[d];
        const float h3 = fmaf(dd[2], 256.0f, fmaf(dd[1], 16.0f, dd[0]));
        // lane groups 0 / 2 hold lo (planes 0..2), 1 / 3 hi (planes 3..5)
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h3), __float_as_uint(h3), false, false);
        P[d] = fmaf(__uint_as_float(sw[1]), 4096.0f, __uint_as_float(sw[0]));
        const uint32_t sbits = __builtin_amdgcn_ubfe(sc[r][slot / 8][slot % 8], ssh, 16u);
        scv[d] = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
        if constexpr (ZK == 1) z[d] = (float)((cb.z[r][d] >> cb.zsh[r][d]) & 3u);
        else if constexpr (ZK == 2) z[d] = (float)cb.zh[r][d];
        else z[d] = zconst;
      }
      if (any_out) {
        // the code of a value taken out of the planes: this lane's own chunk 4u + lg
        // holds it at dword id / 16; lane group 2d + g / 2 owns chunk 4u + 2d + g / 2
        const uint32_t id = __float_as_uint(meta[4 * cit + lg].w);
        const uint32_t di = id >> 4;
        const uint32_t xv = di == 0 ? x.x : di == 1 ? x.y : di == 2 ? x.z : x.w;
        const int own = (int)((xv >> ((id & 15u) * 2u)) & 3u);
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const int slot = 2 * (i % PR) + d;
          const uint32_t code = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (16 * (2 * d + sig) + col), own);
          float t = P[d] * mt[d].x;
          if (mt[d].z != 0.0f) t = fmaf(mt[d].z, (float)code - z[d], t);
          acc[r][slot] = fmaf(scv[d], fmaf(-z[d], mt[d].y, t), acc[r][slot]);
        }
      } else {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const int slot = 2 * (i % PR) + d;
          const float t = P[d] * mt[d].x;
          acc[r][slot] = fmaf(scv[d], fmaf(-z[d], mt[d].y, t), acc[r][slot]);
        }
      }
    }
    if (cit == T2 - 1) {
      // row group complete: partial 2s + c of the v_dot8 kernel is slot s of the
      // lanes of chunk parity c; the butterfly tree pairs 2s with 2s + 1 first
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float e[LPRH];
#pragma unroll
        for (int s = 0; s < LPRH; ++s) e[s] = acc[r][s] + __shfl_xor(acc[r][s], 32, 64);
#pragma unroll
        for (int w = 1; w < LPRH; w *= 2)
#pragma unroll
          for (int s = 0; s < LPRH; s += 2 * w) e[s] = e[s] + e[s + w];
        if (lg == 0) out_lds[(cgrp - g_begin) * rpg + 16 * r + col] = e[0];
#pragma unroll
        for (int s = 0; s < LPRH; ++s) acc[r][s] = 0.0f;
      }
    }
    if (++cit == T2) {
      cit = 0;
      cgrp += NW;
    }
  };

  // rounds of PR pairs: T2 is a multiple of PR, so pair i of a round has slots 2i, 2i + 1
  for (int base = 0; base < total; base += PR) {
#pragma unroll
    for (int i = 0; i < PR; ++i) pair(buf[i % D], buf[(i + D - 1) % D], i);
  }

  __syncthreads();
  const int nrows = (g_end - g_begin) * rpg;
  const int row0 = g_begin * rpg;
  for (int i = threadIdx.x; i < nrows; i += kMxThreads) {
    const int row = row0 + i;
    if (row < N) {
      float v = out_lds[i];
      if (g.bias) v += load_elem_rt(g.bias, g.c_type, row);
      store_elem_rt(g.C, g.c_type, row, v);
    }
  }
}

// Pairs of steps (256 codes) for the matrix-core form, or 0 when the shape does not
// suit it: 2-bit, M = 1, block 64 with a multiple of 8 blocks per row (16-byte scale
// rows), 16 or 32 lanes per row in the v_dot8 kernel, whole rounds, and the operand
// (4 KiB per pair) with its records and row sums within LDS.
inline int gemv_mx_pairs(const GemvArgs& g) {
  if (g.fmt != GEMV_AFFINE || g.bits != 2 || g.M != 1 || !g.chunked || g.block != 64) return 0;
  if (g.nblk % 8 != 0) return 0;
  const int lprh = (1 << g.lpr_log2) / 2;
  if (lprh != 8 && lprh != 16) return 0;
  const int64_t T2 = g.nchunks / 4;
  if (T2 < 1 || T2 % (lprh / 2) != 0) return 0;
  if (g.K * (g.a_type == QMM_F32 ? 4 : 2) >= (1LL << 31) - 64) return 0;
  if ((size_t)T2 * 4096 + (size_t)T2 * 64 + 64 + 16 * 2 * 16 * 4 > kMaxGemvLds) return 0;
  return (int)T2;
}

template <int AT, int R, int LPRH, int ZK>
static hipError_t launch_mx_one(const GemvArgs& g, int T2, hipStream_t st) {
  constexpr int NW = kMxThreads / 64;
  const int64_t rpg = 16 * R;
  // 32-bit buffer offsets for rows up to N plus the groups a fetch runs ahead into
  const int64_t ahead = 2 * (int64_t)NW * rpg;
  if ((g.N + ahead) * g.row_bytes + 64 * (int64_t)T2 >= (1LL << 31) ||
      (g.N + ahead) * g.nblk * 2 + 64 >= (1LL << 31))
    return hipErrorNotSupported;
  const int64_t ngroups = (g.N + rpg - 1) / rpg;
  auto kern = gemv_mx_kernel<AT, R, LPRH, ZK>;
  const size_t base = (size_t)T2 * 4096 + (size_t)T2 * 64 + 64;
  const size_t out_unit = (size_t)rpg * sizeof(float);
  int per_cu = resident_per_cu(kern, kMxThreads, base + (size_t)NW * out_unit);
  int64_t grid = 0, per = 0;
  size_t lds = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t slots = (int64_t)g.num_cus * per_cu;
    grid = slots < ngroups ? slots : ngroups;
    per = (ngroups + grid - 1) / grid;
    lds = base + (size_t)per * out_unit;
    const int again = resident_per_cu(kern, kMxThreads, lds);
    if (again >= per_cu) break;
    per_cu = again;
  }
  if (lds > kMaxGemvLds) return hipErrorNotSupported;
  allow_large_lds(kern, lds);
  launch(kern, dim3((unsigned)grid), dim3(kMxThreads), (uint32_t)lds, st, g, T2);
  return hipSuccess;
}

template <int AT, int LPRH, int ZK>
static hipError_t launch_mx_r(const GemvArgs& g, int R, int T2, hipStream_t st) {
  (void)R;  // one group of 16 rows per wave (two exceed the registers of 16 waves)
  return launch_mx_one<AT, 1, LPRH, ZK>(g, T2, st);
}

// hipErrorNotSupported when the shape does not suit the form.
template <int AT>
hipError_t launch_mx_at_type(const GemvArgs& g, int R, hipStream_t st) {
  const int T2 = gemv_mx_pairs(g);
  if (T2 == 0 || ((uintptr_t)g.scales & 15u) != 0) return hipErrorNotSupported;
  const int zk = g.zp_kind == QMM_ZP_PACKED ? 1 : g.zp_kind == QMM_ZP_F16 ? 2 : 0;
  const int lprh = (1 << g.lpr_log2) / 2;
  if (lprh == 8) {
    if (zk == 1) return launch_mx_r<AT, 8, 1>(g, R, T2, st);
    if (zk == 2) return launch_mx_r<AT, 8, 2>(g, R, T2, st);
    return launch_mx_r<AT, 8, 0>(g, R, T2, st);
  }
  if (zk == 1) return launch_mx_r<AT, 16, 1>(g, R, T2, st);
  if (zk == 2) return launch_mx_r<AT, 16, 2>(g, R, T2, st);
  return launch_mx_r<AT, 16, 0>(g, R, T2, st);
}

}  // namespace qmm
