// Streaming form of the integer-plane GEMV for rows whose activations fit in LDS
// whole (one K-slice).  Same arithmetic and the same summation order as
// gemv_ip_kernel (lanes per row, lane -> chunk map, per-lane chunk order, plane
// sums, fixed xor butterfly), so both give the same bits; this form only removes
// work around the arithmetic:
//   * A is staged once, before the item loop, and the row sums of the whole
//     work-group stay in LDS until one write-out after the loop;
//   * weights, scales and zero points are read with buffer loads whose range
//     check returns 0 past the end, so no address is clamped, and the per-lane
//     offsets advance by a constant per item (no 64-bit address arithmetic);
//   * the loop runs whole rounds of kIpDepth items on scalar counters; every
//     round issues the same loads, so the compiler's memory-counter waits keep
//     kIpDepth - 1 items in flight.
#pragma once
#include "qmm_gemv_ip.h"

namespace qmm {

// Threads per work-group: 16 waves share one copy of the staged activations when
// the kernel's registers allow it (<= 128 VGPRs), else 8.
__host__ __device__ constexpr int stream_threads(int MT, int R) { return MT * R <= 2 ? 1024 : 512; }

template <int BITS, int AT, int MT, int R, int DPG, int ZK>
__global__ __launch_bounds__(stream_threads(MT, R)) void gemv_ip_stream_kernel(GemvArgs g) {
  using L = IpLayout<BITS>;
  constexpr int WPC = 128 / BITS;
  constexpr int G = DPG * L::WPD;  // codes per scale group inside a chunk
  constexpr int NS = 4 / DPG;      // scale groups per chunk
  constexpr int NWAVES = stream_threads(MT, R) / 64;
  constexpr int D = kIpDepth;
  extern __shared__ float lds[];
  const int SC = g.slice_chunks;  // >= nchunks
  uint32_t* planes = (uint32_t*)lds;
  f32x4* meta = (f32x4*)(planes + MT * SC * L::SLOT);
  uint32_t* trash = (uint32_t*)(meta + MT * 4 * SC);  // the 16 floats the plan adds after the records
  float* out_lds = (float*)(trash + 16);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr_log2 = g.lpr_log2;
  const int LPR = 1 << lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> lpr_log2;
  const int SUBS = 64 >> lpr_log2;
  // Row groups (the rows one wave works on at once) are dealt out evenly: work-group
  // b owns the contiguous groups [g_begin, g_end) (counts differ by at most one),
  // and wave w of it takes groups g_begin + w, g_begin + w + NWAVES, ...
  const int rpg = SUBS * R;  // rows per group
  const int N = (int)g.N;
  const int M = (int)g.M;
  const int ngroups = (N + rpg - 1) / rpg;
  const int groups_lo = ngroups / gridDim.x, extra = ngroups % gridDim.x;
  const int g_begin = blockIdx.x * groups_lo + (blockIdx.x < extra ? blockIdx.x : extra);
  const int g_end = g_begin + groups_lo + (blockIdx.x < extra ? 1 : 0);
  if (g_begin >= g_end) return;
  const int wave_groups = g_end - g_begin > wave ? (g_end - g_begin - wave + NWAVES - 1) / NWAVES : 0;
  const int nchunks = (int)g.nchunks;
  const int iters = (nchunks + LPR - 1) >> lpr_log2;  // items per row group
  const int nblk = (int)g.nblk;
  const int blog = g.block_log2;
  const uint32_t row_bytes = (uint32_t)g.row_bytes;
  const float zconst = g.zp_kind == QMM_ZP_UNIFORM ? g.uniform_zp : (float)(1 << (BITS - 1));
  const uint32_t zrow_bytes = (uint32_t)g.zp_row_bytes;
  // scale index of this lane's first group in a chunk of item `it`:
  //   bidx = (it * LPR + lp) * WPC >> blog = it * bstep + lane_b   (it * LPR * WPC is a
  //   multiple of the block: LPR >= 8, WPC >= 32, block <= 256), groups i at + i
  const int bstep = (LPR * WPC) >> blog;
  const int lane_b = (lp * WPC) >> blog;

  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W, (uint32_t)(g.N * g.row_bytes));
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(g.scales, (uint32_t)(g.N * g.nblk * 2));
  __amdgpu_buffer_rsrc_t rZ = rS;
  if constexpr (ZK == 1) rZ = make_rsrc(g.zp, (uint32_t)(g.N * g.zp_row_bytes));
  if constexpr (ZK == 2) rZ = make_rsrc(g.zp, (uint32_t)(g.N * g.nblk * 2));

  // fetch cursor: per-row byte offsets of item 0 of the current group, and the item
  uint32_t fw[R], fs[R], fz[R];
  int fit = 0, fgrp = g_begin + wave;
  auto set_rows = [&](int grp) {
    // Past the wave's own groups (the ring's run-ahead at the end of its work) the
    // cursor moves to group `ngroups`, whose rows all lie past N: rows past N give
    // offsets past the end of every buffer, so those loads return 0 and move no data
    // (the groups that follow belong to the next work-group, whose rows another
    // XCD's L2 reads).
    const int gq = grp < g_end ? grp : ngroups;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = (uint32_t)(gq * rpg + r * SUBS + sub);
      fw[r] = row * row_bytes + (uint32_t)lp * 16u;
      fs[r] = (row * (uint32_t)nblk + (uint32_t)lane_b) * 2u;
      if constexpr (ZK == 1) fz[r] = row * zrow_bytes;
      if constexpr (ZK == 2) fz[r] = fs[r];
    }
  };
  set_rows(fgrp);
  auto fetch = [&](IpBuf<R, NS>& b) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t wo = fw[r] + (uint32_t)(fit * LPR * 16);
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)wo, 0, 0);
      b.w[r] = make_uint4(v[0], v[1], v[2], v[3]);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const uint32_t so = fs[r] + (uint32_t)((fit * bstep + i) * 2);
        b.s[r][i] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rS, (int)so, 0, 0));
        if constexpr (ZK == 1) {
          const int bit = (fit * bstep + lane_b + i) * BITS;
          b.z[r][i] = __builtin_amdgcn_raw_buffer_load_b8(rZ, (int)(fz[r] + (uint32_t)(bit >> 3)), 0, 0);
          b.zsh[r][i] = bit & 7;
        } else if constexpr (ZK == 2) {
          b.zh[r][i] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rZ, (int)so, 0, 0));
        }
      }
    }
    if (++fit == iters) {
      fit = 0;
      fgrp += NWAVES;
      set_rows(fgrp);
    }
  };

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  // the activations' loads go out first, then the first weights of the stream, which
  // travel while the activations are converted
  IpBuf<R, NS> buf[D];
  stage_planes<BITS, AT, G, MT, true>(g, planes, meta, trash, 0, SC, [&] {
#pragma unroll
    for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
  });
  __syncthreads();

  int cit = 0, cgrp = g_begin + wave;
  const int total = wave_groups * iters;
  const uint32_t* planes_lane = planes + lp * L::SLOT;
  const f32x4* meta_lane = meta + lp;
  auto step = [&](IpBuf<R, NS>& cbuf, IpBuf<R, NS>& nxt, bool live) {
    fetch(nxt);
    const int slot = cit * LPR + lp;
    const bool valid = live && slot < nchunks;
    const uint32_t* pb = planes_lane + cit * (LPR * L::SLOT);
    int S[R][MT][6];
    int Sq[R];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (d % DPG == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          Sq[r] = 0;
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int p = 0; p < 6; ++p) S[r][m][p] = 0;
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int mm = m < M ? m : 0;
        const uint32_t* pw = pb + mm * SC * L::SLOT + d * L::PWD;
        uint32_t pl[L::PWD];
        if constexpr (BITS == 2) {
          const uint4 a0 = ((const uint4*)pw)[0], a1 = ((const uint4*)pw)[1], a2 = ((const uint4*)pw)[2];
          pl[0] = a0.x; pl[1] = a0.y; pl[2] = a0.z; pl[3] = a0.w;
          pl[4] = a1.x; pl[5] = a1.y; pl[6] = a1.z; pl[7] = a1.w;
          pl[8] = a2.x; pl[9] = a2.y; pl[10] = a2.z; pl[11] = a2.w;
        } else {
          const uint4 a0 = *(const uint4*)pw;
          const uint2 a1 = *(const uint2*)(pw + 4);
          pl[0] = a0.x; pl[1] = a0.y; pl[2] = a0.z; pl[3] = a0.w;
          pl[4] = a1.x; pl[5] = a1.y;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t x = d == 0 ? cbuf.w[r].x : d == 1 ? cbuf.w[r].y : d == 2 ? cbuf.w[r].z : cbuf.w[r].w;
          if constexpr (BITS == 2) {
            const uint32_t ev = x & 0x33333333u;
            const uint32_t od = (x >> 2) & 0x33333333u;
#pragma unroll
            for (int p = 0; p < 5; ++p) {
              S[r][m][p] = (int)__builtin_amdgcn_udot8(ev, pl[2 * p], (uint32_t)S[r][m][p], false);
              S[r][m][p] = (int)__builtin_amdgcn_udot8(od, pl[2 * p + 1], (uint32_t)S[r][m][p], false);
            }
            S[r][m][5] = __builtin_amdgcn_sdot8((int)ev, (int)pl[10], S[r][m][5], false);
            S[r][m][5] = __builtin_amdgcn_sdot8((int)od, (int)pl[11], S[r][m][5], false);
          } else {
#pragma unroll
            for (int p = 0; p < 6; ++p)
              S[r][m][p] = (int)__builtin_amdgcn_udot8(x, pl[p], (uint32_t)S[r][m][p], false);
            if (m == 0) Sq[r] = (int)__builtin_amdgcn_udot8(x, 0x11111111u, (uint32_t)Sq[r], false);
          }
        }
      }
      if ((d + 1) % DPG == 0) {
        const int gi = d / DPG;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int mm = m < M ? m : 0;
          const f32x4 mt = meta_lane[(mm * 4 + gi) * SC + cit * LPR];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            int s5 = S[r][m][5];
            if constexpr (BITS == 4) s5 -= 8 * Sq[r];  // remove the 2^23 bias of a_int
            const int lo = S[r][m][0] + (S[r][m][1] << 4) + (S[r][m][2] << 8);
            const int hi = S[r][m][3] + (S[r][m][4] << 4) + s5 * 256;
            const float P = fmaf((float)hi, 4096.0f, (float)lo);
            const float scv = (float)cbuf.s[r][gi];
            float z;
            if constexpr (ZK == 1) z = (float)((cbuf.z[r][gi] >> cbuf.zsh[r][gi]) & ((1u << BITS) - 1u));
            else if constexpr (ZK == 2) z = (float)cbuf.zh[r][gi];
            else z = zconst;
            float t = P * mt.x;
            // a value taken out of the planes: a_o * (q_o - zp), q_o - zp exact
            if (mt.z != 0.0f)
              t = fmaf(mt.z, outlier_code<BITS, DPG>(cbuf.w[r], gi, __float_as_uint(mt.w)) - z, t);
            const float nv = fmaf(scv, fmaf(-z, mt.y, t), acc[r][m]);
            acc[r][m] = valid ? nv : acc[r][m];
          }
        }
      }
    }
    if (live && cit == iters - 1) {
      // row group complete: fixed-order combination of the LPR lane partials
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = group_sum(acc[r][m], LPR);
      if (lp == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int lr = (cgrp - g_begin) * rpg + r * SUBS + sub;
#pragma unroll
          for (int m = 0; m < MT; ++m) out_lds[lr * MT + m] = acc[r][m];
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
    }
    if (++cit == iters) {
      cit = 0;
      cgrp += NWAVES;
    }
  };

  for (int base = 0; base < total; base += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) step(buf[i], buf[(i + D - 1) % D], base + i < total);
  }

  // write the row sums (+ bias) of every group of the work-group
  __syncthreads();
  const int nrows = (g_end - g_begin) * rpg;
  const int row0 = g_begin * rpg;
  for (int i = threadIdx.x; i < nrows * M; i += blockDim.x) {
    const int m = i / nrows;
    const int lr = i - m * nrows;
    const int row = row0 + lr;
    if (row < N) {
      float v = out_lds[lr * MT + m];
      if (g.bias) v += load_elem_rt(g.bias, g.c_type, row);
      store_elem_rt(g.C, g.c_type, (int64_t)m * N + row, v);
    }
  }
}

// Launch of the streaming form: one work-group per resident slot (or per row group
// when there are fewer groups), each with an output buffer sized to its rows.
// Returns hipErrorNotSupported when the shape does not suit it (the caller then uses
// gemv_ip_kernel).
template <int BITS, int AT, int MT, int R, int DPG, int ZK>
static hipError_t launch_ip_stream(const GemvArgs& g, hipStream_t st) {
  if (g.slice_chunks < g.nchunks) return hipErrorNotSupported;
  // activations are read with 32-bit buffer offsets
  if (g.M * g.K * (AT == QMM_F32 ? 4 : 2) >= (1LL << 31) - 64) return hipErrorNotSupported;
  // 32-bit buffer offsets: every byte offset below 2^31, for rows up to N plus the
  // groups a wave's fetch may run ahead into (fewer than two work-groups' worth)
  const int64_t rpg = (int64_t)(64 >> g.lpr_log2) * R;
  const int64_t ahead = 2 * (int64_t)(stream_threads(MT, R) / 64) * rpg;
  const int64_t span = (g.N + ahead) * (g.row_bytes + 16 * (1LL << g.lpr_log2));
  if (span >= (1LL << 31) || (g.N + ahead) * g.nblk * 2 >= (1LL << 31)) return hipErrorNotSupported;
  const int64_t ngroups = (g.N + rpg - 1) / rpg;
  auto kern = gemv_ip_stream_kernel<BITS, AT, MT, R, DPG, ZK>;
  const size_t out_unit = (size_t)rpg * MT * sizeof(float);  // per group
  int per_cu = resident_per_cu(kern, stream_threads(MT, R),
                               g.lds_bytes + (size_t)(stream_threads(MT, R) / 64) * out_unit);
  int64_t per = 0, grid = 0;
  size_t lds = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t slots = (int64_t)g.num_cus * per_cu;
    grid = slots < ngroups ? slots : ngroups;  // every resident slot
    per = (ngroups + grid - 1) / grid;         // groups per work-group (at most)
    lds = g.lds_bytes + (size_t)per * out_unit;
    const int again = resident_per_cu(kern, stream_threads(MT, R), lds);
    if (again >= per_cu) break;
    per_cu = again;
  }
  if (lds > kMaxGemvLds) return hipErrorNotSupported;
  allow_large_lds(kern, lds);
  launch(kern, dim3((unsigned)grid), dim3(stream_threads(MT, R)), lds, st, g);
  return hipSuccess;
}

// ---- launch ------------------------------------------------------------------

template <int BITS, int AT, int MT, int R, int DPG, int ZK>
static hipError_t launch_ip_one(const GemvArgs& g, hipStream_t st) {
  const int subs = 64 >> g.lpr_log2;
  const int64_t rows_per_tile = (int64_t)(kGemvThreads / 64) * subs * R;
  const int64_t ntiles = (g.N + rows_per_tile - 1) / rows_per_tile;
  if (launch_ip_stream<BITS, AT, MT, R, DPG, ZK>(g, st) == hipSuccess) return hipSuccess;
  int64_t grid = (int64_t)g.num_cus * g.wg_per_cu;
  if (grid > ntiles) grid = ntiles;
  if (grid < 1) grid = 1;
  const size_t lds = g.lds_bytes + kGemvOutFloats * sizeof(float);
  auto kern = gemv_ip_kernel<BITS, AT, MT, R, DPG, ZK>;
  allow_large_lds(kern, lds);
  launch(kern, dim3((unsigned)grid), dim3(kGemvThreads), lds, st, g);
  return hipSuccess;
}

template <int BITS, int AT, int DPG, int ZK>
static hipError_t launch_ip_mr(const GemvArgs& g, int R, hipStream_t st) {
  switch (g.mt) {
    case 1:
      if (R == 1) return launch_ip_one<BITS, AT, 1, 1, DPG, ZK>(g, st);
      if (R == 2) return launch_ip_one<BITS, AT, 1, 2, DPG, ZK>(g, st);
      return launch_ip_one<BITS, AT, 1, 4, DPG, ZK>(g, st);
    case 2:
      if (R == 1) return launch_ip_one<BITS, AT, 2, 1, DPG, ZK>(g, st);
      return launch_ip_one<BITS, AT, 2, 2, DPG, ZK>(g, st);
    case 4:
      if (R == 1) return launch_ip_one<BITS, AT, 4, 1, DPG, ZK>(g, st);
      return launch_ip_one<BITS, AT, 4, 2, DPG, ZK>(g, st);
    default:
      return launch_ip_one<BITS, AT, 8, 1, DPG, ZK>(g, st);
  }
}

template <int BITS, int AT, int DPG>
static hipError_t launch_ip_zk(const GemvArgs& g, int R, hipStream_t st) {
  if (g.zp_kind == QMM_ZP_PACKED) return launch_ip_mr<BITS, AT, DPG, 1>(g, R, st);
  if (g.zp_kind == QMM_ZP_F16) return launch_ip_mr<BITS, AT, DPG, 2>(g, R, st);
  return launch_ip_mr<BITS, AT, DPG, 0>(g, R, st);
}

template <int BITS, int AT>
hipError_t launch_ip_at_type(const GemvArgs& g, int R, hipStream_t st) {
  constexpr int WPD = 32 / BITS;
  // dwords per scale group: min(block, codes per chunk) / codes per dword
  const int dpg = g.block >= 4 * WPD ? 4 : g.block / WPD;
  if constexpr (BITS == 2) {
    if (dpg == 1) return launch_ip_zk<BITS, AT, 1>(g, R, st);
  }
  if (dpg == 2) return launch_ip_zk<BITS, AT, 2>(g, R, st);
  return launch_ip_zk<BITS, AT, 4>(g, R, st);
}

}  // namespace qmm
