// Streaming form of the codebook GEMV (16-entry table, per-block absmax) for rows
// whose activations fit in LDS whole (one K-slice) and blocks of at least 32 codes
// (one absmax per 16-byte chunk).  Same arithmetic and the same summation order as
// the codebook path of gemv_kernel: the lane -> chunk map and per-lane chunk order,
// eight codes per dword looked up in the LDS table and multiplied into fp32 partials,
// one absmax multiply-add per chunk, and the fixed xor butterfly over the lanes of a
// row.  Both forms therefore give the same bits.  As in the integer-plane streaming
// form, this one only removes work around the arithmetic:
//   * the first weight loads go out, then A is staged once, before the item loop;
//   * weights and absmax come through buffer loads whose range check returns 0 past
//     the end, with per-lane 32-bit offsets that advance by a constant per item;
//   * whole row groups are dealt out evenly over the work-groups, and their row sums
//     stay in LDS until one write-out after the loop.
#pragma once
#include "qmm_gemv_impl.h"
#include "qmm_gemv_stream.h"

namespace qmm {

template <int R>
struct CbBuf {
  uint4 w[R];
  float s[R];
};

template <int AT, int MT, int R>
__global__ __launch_bounds__(stream_threads(MT, R)) void gemv_cb_stream_kernel(GemvArgs g) {
  constexpr int WPC = 32;       // 4-bit codes per 16-byte chunk
  constexpr int WPD = 8;        // codes per dword
  constexpr int CS = WPC + 4;   // LDS floats per chunk slot (the layout of stage_a)
  constexpr int NWAVES = stream_threads(MT, R) / 64;
  constexpr int D = kIpDepth;
  extern __shared__ float lds[];
  // the table sits in static LDS, at an address known when the kernel is built, so a
  // lookup's address is the code's byte offset plus an immediate (no add per code)
  __shared__ float cb_tab[16];
  const int SC = g.slice_chunks;  // >= nchunks
  float* sums_lds = lds + MT * SC * CS;
  float* out_lds = sums_lds + MT * 4 * SC + 16;  // (the plan's 16 spare floats)
  if (threadIdx.x < 16) cb_tab[threadIdx.x] = g.codebook[threadIdx.x];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr_log2 = g.lpr_log2;
  const int LPR = 1 << lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> lpr_log2;
  const int SUBS = 64 >> lpr_log2;
  // work-group b owns the contiguous row groups [g_begin, g_end); wave w of it takes
  // groups g_begin + w, g_begin + w + NWAVES, ...
  const int rpg = SUBS * R;
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
  // absmax index of this lane's chunk in item `it`: (it * LPR + lp) * WPC >> blog
  //   = it * bstep + lane_b (LPR * WPC >= 256 is a multiple of the block)
  const int bstep = (LPR * WPC) >> blog;
  const int lane_b = (lp * WPC) >> blog;

  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.W, (uint32_t)(g.N * g.row_bytes));
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(g.absmax, (uint32_t)(g.N * g.nblk * 4));

  // fetch cursor: per-row byte offsets of item 0 of the current group, and the item
  uint32_t fw[R], fs[R];
  int fit = 0, fgrp = g_begin + wave;
  auto set_rows = [&](int grp) {
    // past the wave's own groups the cursor moves to group `ngroups`, whose rows lie
    // past N: offsets past the end of both buffers, loads that return 0 and move no data
    const int gq = grp < g_end ? grp : ngroups;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = (uint32_t)(gq * rpg + r * SUBS + sub);
      fw[r] = row * row_bytes + (uint32_t)lp * 16u;
      fs[r] = (row * (uint32_t)nblk + (uint32_t)lane_b) * 4u;
    }
  };
  set_rows(fgrp);
  auto fetch = [&](CbBuf<R>& b) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t wo = fw[r] + (uint32_t)(fit * LPR * 16);
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)wo, 0, 0);
      b.w[r] = make_uint4(v[0], v[1], v[2], v[3]);
      const uint32_t so = fs[r] + (uint32_t)(fit * bstep * 4);
      b.s[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, (int)so, 0, 0));
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

  // the first weights of the stream travel while the activations are staged
  CbBuf<R> buf[D];
#pragma unroll
  for (int i = 0; i < D - 1; ++i) fetch(buf[i]);
  stage_a<AT, WPC, CS>(g, lds, sums_lds, 0, SC, WPC);
  __syncthreads();

  int cit = 0, cgrp = g_begin + wave;
  const int total = wave_groups * iters;
  auto step = [&](CbBuf<R>& cbuf, CbBuf<R>& nxt, bool live) {
    fetch(nxt);
    const int slot = cit * LPR + lp;
    const bool valid = live && slot < nchunks;
    const float* abase = lds + slot * CS;
    float P[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) P[r][m] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float a[MT][WPD];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int mm = m < M ? m : 0;
        const f32x4* ap = (const f32x4*)(abase + mm * SC * CS + d * WPD);
        const f32x4 v0 = ap[0], v1 = ap[1];
        a[m][0] = v0.x; a[m][1] = v0.y; a[m][2] = v0.z; a[m][3] = v0.w;
        a[m][4] = v1.x; a[m][5] = v1.y; a[m][6] = v1.z; a[m][7] = v1.w;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t x = d == 0 ? cbuf.w[r].x : d == 1 ? cbuf.w[r].y : d == 2 ? cbuf.w[r].z : cbuf.w[r].w;
        float q[WPD];
        const uint32_t lo4 = (x << 2) & 0x3c3c3c3cu;  // byte b = 4 * code(2b)
        const uint32_t hi4 = (x >> 2) & 0x3c3c3c3cu;  // byte b = 4 * code(2b+1)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          q[2 * b + 0] = cb_tab[__builtin_amdgcn_ubfe(lo4, 8 * b, 8) >> 2];
          q[2 * b + 1] = cb_tab[__builtin_amdgcn_ubfe(hi4, 8 * b, 8) >> 2];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int i = 0; i < WPD; ++i) P[r][m] = fmaf(a[m][i], q[i], P[r][m]);
      }
    }
    // the chunk is one scale group: one absmax multiply-add per row and A row
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float nv = fmaf(cbuf.s[r], P[r][m], acc[r][m]);
        acc[r][m] = valid ? nv : acc[r][m];
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

// The kernel's static table takes 64 bytes of the work-group's LDS, so its dynamic
// LDS may reach the CU's limit less those.
constexpr size_t kCbStaticLds = 16 * sizeof(float);

template <typename K>
static void allow_cb_lds(K kern, size_t lds) {
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(kMaxGemvLds - kCbStaticLds));
}

// Work-groups of `kern` with `lds` bytes of dynamic LDS resident on one compute unit,
// cached per (kernel, LDS size).
template <typename K>
static int cb_resident_per_cu(K kern, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<const void*, size_t>, int> cache;
  const auto key = std::make_pair((const void*)kern, lds);
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  allow_cb_lds(kern, lds);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, lds) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = n;
  return n;
}

// Launch of the streaming form: one work-group per resident slot (or per row group
// when there are fewer groups), each with an output buffer sized to its rows.
// Returns hipErrorNotSupported when the shape does not suit it.
template <int AT, int MT, int R>
static hipError_t launch_cb_stream(const GemvArgs& g, hipStream_t st) {
  if (g.slice_chunks < g.nchunks || g.block < 32) return hipErrorNotSupported;
  // 32-bit buffer offsets: every byte offset below 2^31, for rows up to N plus the
  // groups a wave's fetch may run ahead into (fewer than two work-groups' worth)
  const int64_t rpg = (int64_t)(64 >> g.lpr_log2) * R;
  const int64_t ahead = 2 * (int64_t)(stream_threads(MT, R) / 64) * rpg;
  const int64_t span = (g.N + ahead) * (g.row_bytes + 16 * (1LL << g.lpr_log2));
  if (span >= (1LL << 31) || (g.N + ahead) * (g.nblk + (1LL << g.lpr_log2)) * 4 >= (1LL << 31))
    return hipErrorNotSupported;
  const int64_t ngroups = (g.N + rpg - 1) / rpg;
  auto kern = gemv_cb_stream_kernel<AT, MT, R>;
  const size_t out_unit = (size_t)rpg * MT * sizeof(float);  // per group
  int per_cu = cb_resident_per_cu(kern, stream_threads(MT, R),
                                  g.lds_bytes + (size_t)(stream_threads(MT, R) / 64) * out_unit);
  int64_t grid = 0;
  size_t lds = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t slots = (int64_t)g.num_cus * per_cu;
    grid = slots < ngroups ? slots : ngroups;       // every resident slot
    const int64_t per = (ngroups + grid - 1) / grid;  // groups per work-group (at most)
    lds = g.lds_bytes + (size_t)per * out_unit;
    const int again = cb_resident_per_cu(kern, stream_threads(MT, R), lds);
    if (again >= per_cu) break;
    per_cu = again;
  }
  if (lds + kCbStaticLds > kMaxGemvLds) return hipErrorNotSupported;
  allow_cb_lds(kern, lds);
  launch(kern, dim3((unsigned)grid), dim3(stream_threads(MT, R)), lds, st, g);
  return hipSuccess;
}

template <int AT, int MT, int R>
static hipError_t launch_cb_one(const GemvArgs& g, hipStream_t st) {
  if (launch_cb_stream<AT, MT, R>(g, st) == hipSuccess) return hipSuccess;
  return g.block < 32 ? launch_one<GEMV_CODEBOOK, 4, AT, MT, R, 1, 0>(g, st)
                      : launch_one<GEMV_CODEBOOK, 4, AT, MT, R, 0, 0>(g, st);
}

// Codebook GEMV for one activation type: the streaming form where it applies, else
// gemv_kernel (same bits either way).
template <int AT>
hipError_t launch_cb_at_type(const GemvArgs& g, int R, hipStream_t st) {
  switch (g.mt) {
    case 1:
      if (R == 1) return launch_cb_one<AT, 1, 1>(g, st);
      if (R == 2) return launch_cb_one<AT, 1, 2>(g, st);
      return launch_cb_one<AT, 1, 4>(g, st);
    case 2:
      if (R == 1) return launch_cb_one<AT, 2, 1>(g, st);
      return launch_cb_one<AT, 2, 2>(g, st);
    case 4:
      if (R == 1) return launch_cb_one<AT, 4, 1>(g, st);
      return launch_cb_one<AT, 4, 2>(g, st);
    default:
      return launch_cb_one<AT, 8, 1>(g, st);
  }
}

}  // namespace qmm
