// Weight-streaming GEMV / skinny GEMM for M <= 8 on gfx950.
//
// Affine MatMulNBits weights ([P1] hip-ep PR 1318, "What", commit 1: GEMV that reads
// fp32 A and writes fp32 C directly; uniform zero point as a scalar) and 16-entry
// codebook 4-bit weights ([P3] bitsandbytes PR 1979, "Technical details": centroids
// staged in LDS, scale applied once per chunk, next chunk prefetched into registers).
//
// Work decomposition (fixed by K, block and bits only, so every tiling gives the
// same bits):
//   * a weight row is read as 16-byte chunks; chunk c holds WPC = 128/bits codes;
//   * each row is owned by a group of LPR lanes (LPR in {8,16,32,64}, chosen from
//     the chunk count); lane p of the group handles chunks p, p+LPR, ... in order;
//   * inside a chunk the codes are decoded four bytes at a time and multiplied into
//     a per-group partial sum in index order; the group's scale (and zero point,
//     folded as s * (sum a*q - zp * sum a)) is applied once per block group;
//   * the LPR lane partials are combined by a fixed xor butterfly.
// A tile of R rows per lane (the tunable part) only changes which wave owns a row.
#pragma once
#include "qmm_device.h"
#include "qmm_internal.h"

#include <map>
#include <mutex>
#include <utility>

namespace qmm {

// --- decoding four bytes (one dword) of codes into fp32 ------------------------
//
// 2-bit codes: masking with 0x33333333 leaves codes 4b and 4b+2 of byte b as the
// two nibbles of that byte, each in 0..3; as e2m1 (fp4) nibbles 0..3 decode to
// 0, 0.5, 1, 1.5, i.e. exactly q/2, two at a time with one conversion.
// 4-bit codes: masking with 0x0f0f0f0f leaves one code per byte; as e4m3 (fp8)
// bytes 0..15 decode to exactly q * 2^-9, two at a time.
template <int B>
__device__ __forceinline__ void fp4_pair(uint32_t ev, uint32_t od, float (&q)[16]) {
  f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, B);
  f32x2 o = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, B);
  q[4 * B + 0] = e.x;
  q[4 * B + 2] = e.y;
  q[4 * B + 1] = o.x;
  q[4 * B + 3] = o.y;
}

template <int BITS>
__device__ __forceinline__ void decode_dword_affine(uint32_t x, float (&q)[32 / BITS]) {
  if constexpr (BITS == 2) {
    const uint32_t ev = x & 0x33333333u;
    const uint32_t od = (x >> 2) & 0x33333333u;
    fp4_pair<0>(ev, od, q);
    fp4_pair<1>(ev, od, q);
    fp4_pair<2>(ev, od, q);
    fp4_pair<3>(ev, od, q);
  } else {
    const uint32_t lo = x & 0x0f0f0f0fu;
    const uint32_t hi = (x >> 4) & 0x0f0f0f0fu;
    f32x2 l0 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
    f32x2 l1 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    f32x2 h0 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    f32x2 h1 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    q[0] = l0.x; q[2] = l0.y; q[4] = l1.x; q[6] = l1.y;
    q[1] = h0.x; q[3] = h0.y; q[5] = h1.x; q[7] = h1.y;
  }
}

// Factor that turns the decoded values above into the codes themselves (3- and 8-bit
// codes are decoded as the codes).
template <int BITS>
__device__ __forceinline__ constexpr float affine_decode_factor() {
  return BITS == 2 ? 2.0f : BITS == 4 ? 512.0f : 1.0f;
}

// Bytes of one weight chunk of a lane: 16 (64 u2, 32 u4, 16 i8 codes) or 12 for 3-bit
// codes (32 codes: a 16-byte chunk would split a code).
template <int BITS>
__host__ __device__ __forceinline__ constexpr int chunk_bytes() {
  return BITS == 3 ? 12 : 16;
}

// Codes [8d, 8d + 8) of a 12-byte chunk of 3-bit codes (24 bits at bit 24d), as floats.
__device__ __forceinline__ void decode_group_u3(const uint4& w, int d, float (&q)[8]) {
  const uint32_t x = d == 0 ? w.x : d == 1 ? __builtin_amdgcn_alignbit(w.y, w.x, 24)
                   : d == 2 ? __builtin_amdgcn_alignbit(w.z, w.y, 16) : (w.z >> 8);
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = (float)__builtin_amdgcn_ubfe(x, 3 * i, 3);
}

// The four signed 8-bit codes of a dword, as floats.
__device__ __forceinline__ void decode_dword_i8(uint32_t x, float (&q)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = (float)(int)__builtin_amdgcn_sbfe((int)x, 8 * i, 8);
}

// The weight chunk of one lane: 16 bytes, or 12 for 3-bit codes (w.w unused).
template <int BITS>
__device__ __forceinline__ uint4 load_chunk(const uint8_t* p) {
  if constexpr (BITS == 3) {
    const uint32_t* q = (const uint32_t*)p;
    return make_uint4(q[0], q[1], q[2], 0u);
  } else {
    return *(const uint4*)p;
  }
}

// Packed zero-point code `idx` of a row (the weights' field layout; signed for 8 bits).
template <int BITS>
__device__ __forceinline__ float packed_zp_code(const uint8_t* row, int idx) {
  if constexpr (BITS == 8) return (float)(int8_t)row[idx];
  const int bit = idx * BITS;
  uint32_t v = row[bit >> 3];
  if ((bit & 7) + BITS > 8) v |= (uint32_t)row[(bit >> 3) + 1] << 8;
  return (float)((v >> (bit & 7)) & ((1u << BITS) - 1u));
}

// Codebook lookup of the eight 4-bit codes of a dword from the LDS table.
__device__ __forceinline__ void decode_dword_codebook(uint32_t x, const float* cb, float (&q)[8]) {
  const uint32_t lo4 = (x << 2) & 0x3c3c3c3cu;  // byte b = 4 * code(2b)
  const uint32_t hi4 = (x >> 2) & 0x3c3c3c3cu;  // byte b = 4 * code(2b+1)
  const char* base = (const char*)cb;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    q[2 * b + 0] = *(const float*)(base + __builtin_amdgcn_ubfe(lo4, 8 * b, 8));
    q[2 * b + 1] = *(const float*)(base + __builtin_amdgcn_ubfe(hi4, 8 * b, 8));
  }
}

// Stage the activations of chunks [c0, c0 + SC) of every A row into LDS as fp32:
// chunk slot `slot` of row m occupies lds[(m * SC + slot) * CS .. + WPC); codes past
// K read 0 (the 4 padding floats per slot spread the lanes of a wave over distinct
// LDS banks).  The sums of A over each scale group of G codes, used by the zero
// point fold, go to sums[(m * 4 + gi) * SC + slot]; each is reduced over the G/4
// threads that staged it by a fixed xor butterfly.
template <int AT, int WPC, int CS>
__device__ __forceinline__ void stage_a(const GemvArgs& g, float* lds, float* sums, int c0, int SC,
                                        int G) {
  const int per_row = SC * (WPC / 4);  // float4 pieces per A row in the slice
  const int total = (int)g.M * per_row;
  const int K = (int)g.K;
  const int gw = G / 4;  // threads per scale group (4, 8 or 16; aligned groups of lanes)
  for (int base_idx = 0; base_idx < total; base_idx += blockDim.x) {
    const int idx = base_idx + threadIdx.x;
    const bool ok = idx < total;
    const int m = ok ? idx / per_row : 0;
    const int rem = idx - m * per_row;
    const int slot = rem / (WPC / 4);
    const int j4 = rem - slot * (WPC / 4);
    const int k = (c0 + slot) * WPC + 4 * j4;
    const int64_t base = (int64_t)m * K + k;
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
      if (g.a_vec && k + 3 < K) {
        if constexpr (AT == QMM_F32) {
          v = *(const f32x4*)((const float*)g.A + base);
        } else {
          const uint2 u = *(const uint2*)((const uint16_t*)g.A + base);
          if constexpr (AT == QMM_F16) {
            v.x = f16_to_f32((uint16_t)(u.x & 0xffffu));
            v.y = f16_to_f32((uint16_t)(u.x >> 16));
            v.z = f16_to_f32((uint16_t)(u.y & 0xffffu));
            v.w = f16_to_f32((uint16_t)(u.y >> 16));
          } else {
            v.x = __uint_as_float(u.x << 16);
            v.y = __uint_as_float(u.x & 0xffff0000u);
            v.z = __uint_as_float(u.y << 16);
            v.w = __uint_as_float(u.y & 0xffff0000u);
          }
        }
      } else {
        v.x = (k + 0 < K) ? load_elem<AT>(g.A, base + 0) : 0.0f;
        v.y = (k + 1 < K) ? load_elem<AT>(g.A, base + 1) : 0.0f;
        v.z = (k + 2 < K) ? load_elem<AT>(g.A, base + 2) : 0.0f;
        v.w = (k + 3 < K) ? load_elem<AT>(g.A, base + 3) : 0.0f;
      }
      *(f32x4*)(lds + (m * SC + slot) * CS + 4 * j4) = v;
    }
    float part = ((v.x + v.y) + v.z) + v.w;
    for (int off = 1; off < gw; off <<= 1) part += __shfl_xor(part, off, 64);
    if (ok && (j4 % gw) == 0) sums[(m * 4 + j4 / gw) * SC + slot] = part;
  }
}

// Weights and scale data of one work item of one lane: R rows x one 16-byte chunk,
// plus NS = 1 (or 4 when a chunk spans several blocks) scales and zero points per row.
template <int R, int NS>
struct ItemBuf {
  uint4 w[R];
  float s[R][NS];
  float z[R][NS];
};

constexpr int kGemvThreads = 512;     // 8 waves per work-group
constexpr int kGemvDepth = 3;         // items per lane whose loads are in flight
constexpr int kGemvOutFloats = 4096;  // LDS output buffer (flushed when full)

// Position of a lane in the item sequence of its work-group.
struct ItemPos {
  int tile, s, it;
};

// Persistent weight-streaming kernel.  Work-group g owns the contiguous tiles
// [t_begin, t_end) of 8*SUBS*R rows each; every lane walks the sequence (tile,
// K-slice, chunk iteration) with the loads of the next kGemvDepth-1 items in
// flight in a ring of register sets (the loop is unrolled kGemvDepth times so
// the sets rotate without copies; every fetch issues the same loads, with
// clamped addresses past the end, so the compiler's wait counts stay exact).
// Finished row sums go to an LDS buffer that is written out with coalesced
// stores only when full and at the end, so no store or bias load sits between a
// prefetch and its use.  A is staged in LDS one K-slice of SC chunks at a time
// (once per work-group when one slice covers K).
// ZK: 0 = zero point is a constant (none / uniform), 1 = packed codes, 2 = fp16
// tensor.  MULTI: a chunk spans several blocks (block < codes per chunk).
template <int FMT, int BITS, int AT, int MT, int R, int MULTI, int ZK>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs g) {
  constexpr int CHB = chunk_bytes<BITS>();
  constexpr int WPC = CHB * 8 / BITS;  // codes per chunk
  constexpr int WPD = WPC / 4;         // codes per decode step (a dword, or 24 bits of u3)
  constexpr int CS = WPC + 4;          // LDS floats per chunk slot
  constexpr int NS = MULTI ? 4 : 1;
  constexpr int D = kGemvDepth;
  constexpr int NWAVES = kGemvThreads / 64;
  extern __shared__ float lds[];
  const int SC = g.slice_chunks;
  float* sums_lds = lds + MT * SC * CS;
  float* cb_lds = sums_lds + MT * 4 * SC;
  float* out_lds = cb_lds + 16;
  if constexpr (FMT == GEMV_CODEBOOK) {
    if (threadIdx.x < 16) cb_lds[threadIdx.x] = g.codebook[threadIdx.x];
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lpr_log2 = g.lpr_log2;
  const int LPR = 1 << lpr_log2;
  const int lp = lane & (LPR - 1);
  const int sub = lane >> lpr_log2;
  const int SUBS = 64 >> lpr_log2;
  const int rows_per_wave = SUBS * R;
  const int rows_per_tile = NWAVES * rows_per_wave;
  const int N = (int)g.N;
  const int M = (int)g.M;
  const int ntiles = (N + rows_per_tile - 1) / rows_per_tile;
  // contiguous tile range of this work-group
  const int tiles_lo = ntiles / gridDim.x, extra = ntiles % gridDim.x;
  const int t_begin = blockIdx.x * tiles_lo + (blockIdx.x < extra ? blockIdx.x : extra);
  const int t_end = t_begin + tiles_lo + (blockIdx.x < extra ? 1 : 0);
  if (t_begin >= t_end) return;
  const int nchunks = (int)g.nchunks;
  const int nslices = (nchunks + SC - 1) / SC;
  const int iters = SC >> lpr_log2;  // chunk iterations per slice
  const int nblk = (int)g.nblk;
  const int blog = g.block_log2;
  const int G = g.block < WPC ? g.block : WPC;  // codes per scale group inside a chunk
  const int GPC = WPC / G;                       // groups per chunk: 1, 2 or 4
  const int DPG = G / WPD;                       // dwords per group: 1, 2 or 4
  const int64_t row_bytes = g.row_bytes;
  constexpr float FAC = (FMT == GEMV_AFFINE) ? affine_decode_factor<BITS>() : 1.0f;
  const float zconst = g.zp_kind == QMM_ZP_UNIFORM ? g.uniform_zp : default_zero_point(BITS);
  const int zrow_bytes = (int)g.zp_row_bytes;
  // output buffer: tiles per flush
  int out_tiles = kGemvOutFloats / (rows_per_tile * MT);
  if (out_tiles < 1) out_tiles = 1;

  auto advance = [&](ItemPos& p) {
    if (++p.it == iters) {
      p.it = 0;
      if (++p.s == nslices) {
        p.s = 0;
        ++p.tile;
      }
    }
  };
  // fetch cursor: the next item to load, its chunk, and the row bases of its tile
  ItemPos fpos{t_begin, 0, 0};
  int fchunk = lp;  // chunk of this lane in the item at fpos
  const uint8_t* fw[R];
  const uint16_t* fsa[R];    // affine scales row
  const float* fab[R];       // codebook absmax row
  const uint8_t* fzp[R];     // packed zero-point row
  const uint16_t* fzh[R];    // fp16 zero-point row
  auto set_bases = [&](int tl) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int row = tl * rows_per_tile + wave * rows_per_wave + r * SUBS + sub;
      row = (tl < t_end && row < N) ? row : N - 1;
      fw[r] = g.W + (int64_t)row * row_bytes;
      if constexpr (FMT == GEMV_AFFINE) fsa[r] = g.scales + (int64_t)row * nblk;
      else fab[r] = g.absmax + (int64_t)row * nblk;
      if constexpr (ZK == 1) fzp[r] = (const uint8_t*)g.zp + (int64_t)row * zrow_bytes;
      if constexpr (ZK == 2) fzh[r] = (const uint16_t*)g.zp + (int64_t)row * nblk;
    }
  };
  set_bases(t_begin);
  // load the item at the fetch cursor into b and advance the cursor: always the same
  // loads; past the end of the work the last row / chunk is read (results unused)
  auto fetch_next = [&](ItemBuf<R, NS>& b) {
    const int cc = (fpos.tile < t_end && fchunk < nchunks) ? fchunk : nchunks - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      b.w[r] = load_chunk<BITS>(fw[r] + cc * CHB);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int gi = i < GPC ? i : GPC - 1;
        const int bidx = (cc * WPC + gi * G) >> blog;
        if constexpr (FMT == GEMV_AFFINE) {
          b.s[r][i] = f16_to_f32(fsa[r][bidx]);
          if constexpr (ZK == 1) {
            b.z[r][i] = packed_zp_code<BITS>(fzp[r], bidx);
          } else if constexpr (ZK == 2) {
            b.z[r][i] = f16_to_f32(fzh[r][bidx]);
          } else {
            b.z[r][i] = zconst;
          }
        } else {
          b.s[r][i] = fab[r][bidx];
          b.z[r][i] = 0.0f;
        }
      }
    }
    const int old_tile = fpos.tile;
    advance(fpos);
    if (fpos.tile != old_tile) {
      fchunk = lp;
      set_bases(fpos.tile);
    } else {
      fchunk = fpos.s * SC + fpos.it * LPR + lp;
    }
  };
  // write the buffered row sums of tiles [tf, tl) (+ bias) to C
  auto flush = [&](int tf, int tl) {
    __syncthreads();
    const int nrows = (tl - tf) * rows_per_tile;
    const int row0 = tf * rows_per_tile;
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
    __syncthreads();
  };

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  ItemPos cur{t_begin, 0, 0};   // item being computed
  bool staged = false;
  int flush_from = t_begin;
  bool done = false;

  // One step: stage A if this item starts a slice, fetch the item D-1 ahead into
  // `nxt` (the set that held the previous item), compute the current item from
  // `cb`, and finish the tile if it ends here.
  auto step = [&](ItemBuf<R, NS>& cbuf, ItemBuf<R, NS>& nxt) {
    if (cur.it == 0 && (nslices > 1 || !staged)) {
      __syncthreads();
      stage_a<AT, WPC, CS>(g, lds, sums_lds, cur.s * SC, SC, G);
      __syncthreads();
      staged = true;
    }
    fetch_next(nxt);

    const int c = cur.s * SC + cur.it * LPR + lp;
    if (c < nchunks) {
      const float* abase = lds + (cur.it * LPR + lp) * CS;
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
#pragma unroll
          for (int i = 0; i < WPD / 4; ++i) {
            const f32x4 v = ap[i];
            a[m][4 * i + 0] = v.x; a[m][4 * i + 1] = v.y; a[m][4 * i + 2] = v.z; a[m][4 * i + 3] = v.w;
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t x = d == 0 ? cbuf.w[r].x : d == 1 ? cbuf.w[r].y : d == 2 ? cbuf.w[r].z : cbuf.w[r].w;
          float q[WPD];
          if constexpr (FMT == GEMV_CODEBOOK) decode_dword_codebook(x, cb_lds, q);
          else if constexpr (BITS == 3) decode_group_u3(cbuf.w[r], d, q);
          else if constexpr (BITS == 8) decode_dword_i8(x, q);
          else decode_dword_affine<BITS>(x, q);
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < WPD; ++i) P[r][m] = fmaf(a[m][i], q[i], P[r][m]);
        }
        if (!MULTI ? d == 3 : (((d + 1) % DPG) == 0)) {
          // scale group gi of the chunk complete
          const int gi = MULTI ? d / DPG : 0;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float scv, z;
            if constexpr (MULTI) {
              scv = gi == 0 ? cbuf.s[r][0] : gi == 1 ? cbuf.s[r][NS > 1 ? 1 : 0]
                  : gi == 2 ? cbuf.s[r][NS > 2 ? 2 : 0] : cbuf.s[r][NS > 3 ? 3 : 0];
              z = gi == 0 ? cbuf.z[r][0] : gi == 1 ? cbuf.z[r][NS > 1 ? 1 : 0]
                  : gi == 2 ? cbuf.z[r][NS > 2 ? 2 : 0] : cbuf.z[r][NS > 3 ? 3 : 0];
            } else {
              scv = cbuf.s[r][0];
              z = cbuf.z[r][0];
            }
            if constexpr (FMT == GEMV_AFFINE) {
#pragma unroll
              for (int m = 0; m < MT; ++m) {
                const int mm = m < M ? m : 0;
                const float sa = sums_lds[(mm * 4 + gi) * SC + cur.it * LPR + lp];
                acc[r][m] = fmaf(scv, fmaf(-z, sa, FAC * P[r][m]), acc[r][m]);
                P[r][m] = 0.0f;
              }
            } else {
#pragma unroll
              for (int m = 0; m < MT; ++m) {
                acc[r][m] = fmaf(scv, P[r][m], acc[r][m]);
                P[r][m] = 0.0f;
              }
            }
          }
        }
      }
    }

    if (cur.s == nslices - 1 && cur.it == iters - 1) {
      // tile complete: fixed-order combination of the LPR lane partials of each row
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = group_sum(acc[r][m], LPR);
      if (lp == 0) {
        const int lt = cur.tile - flush_from;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int lr = lt * rows_per_tile + wave * rows_per_wave + r * SUBS + sub;
#pragma unroll
          for (int m = 0; m < MT; ++m) out_lds[lr * MT + m] = acc[r][m];
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
      if (cur.tile + 1 == t_end || cur.tile + 1 - flush_from == out_tiles) {
        flush(flush_from, cur.tile + 1);
        flush_from = cur.tile + 1;
      }
      done = cur.tile + 1 == t_end;
    }
    advance(cur);
  };

  ItemBuf<R, NS> b0, b1, b2;
  static_assert(D == 3, "the unrolled loop below rotates three register sets");
  fetch_next(b0);
  fetch_next(b1);
  while (true) {
    step(b0, b2);
    if (done) break;
    step(b1, b0);
    if (done) break;
    step(b2, b1);
    if (done) break;
  }
}

// ---- launch ------------------------------------------------------------------

template <typename K>
static void allow_large_lds(K kernel, size_t lds) {
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kMaxGemvLds);
}

// Work-groups of `kern` (`threads` threads, `lds` bytes of dynamic LDS) that can be
// resident on one compute unit; cached per (kernel, LDS size).
template <typename K>
static int resident_per_cu(K kern, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<const void*, size_t>, int> cache;
  const auto key = std::make_pair((const void*)kern, lds);
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  allow_large_lds(kern, lds);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, lds) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = n;
  return n;
}

template <int FMT, int BITS, int AT, int MT, int R, int MULTI, int ZK>
static hipError_t launch_one(const GemvArgs& g, hipStream_t st) {
  const int subs = 64 >> g.lpr_log2;
  const int64_t rows_per_tile = (int64_t)(kGemvThreads / 64) * subs * R;
  const int64_t ntiles = (g.N + rows_per_tile - 1) / rows_per_tile;
  int64_t grid = (int64_t)g.num_cus * g.wg_per_cu;
  if (grid > ntiles) grid = ntiles;
  if (grid < 1) grid = 1;
  const size_t lds = g.lds_bytes + kGemvOutFloats * sizeof(float);
  auto kern = gemv_kernel<FMT, BITS, AT, MT, R, MULTI, ZK>;
  allow_large_lds(kern, lds);
  launch(kern, dim3((unsigned)grid), dim3(kGemvThreads), lds, st, g);
  return hipSuccess;
}

template <int FMT, int BITS, int AT, int MULTI, int ZK>
static hipError_t launch_mr(const GemvArgs& g, int R, hipStream_t st) {
  switch (g.mt) {
    case 1:
      if (R == 1) return launch_one<FMT, BITS, AT, 1, 1, MULTI, ZK>(g, st);
      if (R == 2) return launch_one<FMT, BITS, AT, 1, 2, MULTI, ZK>(g, st);
      return launch_one<FMT, BITS, AT, 1, 4, MULTI, ZK>(g, st);
    case 2:
      if (R == 1) return launch_one<FMT, BITS, AT, 2, 1, MULTI, ZK>(g, st);
      return launch_one<FMT, BITS, AT, 2, 2, MULTI, ZK>(g, st);
    case 4:
      if (R == 1) return launch_one<FMT, BITS, AT, 4, 1, MULTI, ZK>(g, st);
      return launch_one<FMT, BITS, AT, 4, 2, MULTI, ZK>(g, st);
    default:
      return launch_one<FMT, BITS, AT, 8, 1, MULTI, ZK>(g, st);
  }
}

template <int FMT, int BITS, int AT>
hipError_t launch_at_type(const GemvArgs& g, int R, hipStream_t st) {
  constexpr int WPC = chunk_bytes<BITS>() * 8 / BITS;
  const bool multi = g.block < WPC;
  if constexpr (FMT == GEMV_CODEBOOK) {
    return multi ? launch_mr<FMT, BITS, AT, 1, 0>(g, R, st) : launch_mr<FMT, BITS, AT, 0, 0>(g, R, st);
  } else {
    const int zk = g.zp_kind == QMM_ZP_PACKED ? 1 : g.zp_kind == QMM_ZP_F16 ? 2 : 0;
    if (multi) {
      if (zk == 1) return launch_mr<FMT, BITS, AT, 1, 1>(g, R, st);
      if (zk == 2) return launch_mr<FMT, BITS, AT, 1, 2>(g, R, st);
      return launch_mr<FMT, BITS, AT, 1, 0>(g, R, st);
    }
    if (zk == 1) return launch_mr<FMT, BITS, AT, 0, 1>(g, R, st);
    if (zk == 2) return launch_mr<FMT, BITS, AT, 0, 2>(g, R, st);
    return launch_mr<FMT, BITS, AT, 0, 0>(g, R, st);
  }
}

}  // namespace qmm
