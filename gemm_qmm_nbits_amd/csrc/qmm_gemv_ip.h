// Weight-streaming GEMV for affine 2-bit / 4-bit MatMulNBits weights with exact
// integer dot products ([P1] hip-ep PR 1318, "What", commit 1: a GEMV that reads
// fp32 A directly; zero point folded so a uniform zero point costs nothing).
//
// Each scale group of G codes of A (G = min(block, codes per 16-byte chunk)) is
// staged in LDS as a block fixed-point number: a_int = rint(a * 2^(22 - e)) with
// 2^e > max |a| over the group (so |a_int| <= 2^22 and the rounding error is at most
// 2^-23 of the group maximum), stored as six 4-bit planes.  The dot product of a
// chunk of codes with one plane is then exact in int32 with v_dot8 (eight 4-bit
// products per instruction):
//   2-bit codes: masking the weight dword with 0x33333333 (and the dword shifted
//     right by 2) leaves the even (odd) codes as nibbles in index order; the A
//     planes hold the digits of the even / odd activations in the same order; the
//     top plane is the signed top nibble of a_int (sdot8; codes 0..3 are also valid
//     signed nibbles), the other five are unsigned (udot8).
//   4-bit codes: the weight dword already holds eight codes as nibbles; the planes
//     hold the digits of a_int + 2^23 (all unsigned), and the bias is removed
//     exactly from the top plane's sum with sum(q) (udot8 against 0x11111111).
// Per group and row:  P = sum_k a_int[k] q[k]  (planes combined in int32 and one
// fp32 multiply-add), and the row partial gains  s * (P * 2^(e-22) - zp * sum_k a[k])
// where sum_k a[k] is the fp32 group sum taken at staging.
//
// The work decomposition (lanes per row, lane -> chunk map, per-lane chunk order,
// fixed xor butterfly, tiles, prefetch ring, LDS output buffer) is that of the
// fp32 kernel in qmm_gemv_impl.h, so the summation order again depends only on
// (K, block, bits).
#pragma once
#include "qmm_gemv_impl.h"

namespace qmm {

#ifndef QMM_IP_DEPTH
#define QMM_IP_DEPTH 2
#endif
constexpr int kIpDepth = QMM_IP_DEPTH;  // items per lane whose loads are in flight

// Raw loads of one work item of one lane: R rows x one 16-byte chunk, NS scales and
// zero points per row.  They are kept as loaded and decoded where they are used,
// so nothing between a prefetch and its use has to wait for the load.
template <int R, int NS>
struct IpBuf {
  uint4 w[R];
  _Float16 s[R][NS];    // scale
  _Float16 zh[R][NS];   // fp16 zero point
  uint32_t z[R][NS];    // packed zero-point byte
  uint32_t zsh[R][NS];  // bit offset of the code in the packed zero-point byte
};

// LDS words of A planes per 16-byte chunk slot (padded so consecutive slots start
// in different bank groups) and per dword of weights.
template <int BITS>
struct IpLayout {
  static constexpr int WPD = 32 / BITS;                // codes per weight dword
  static constexpr int PWD = BITS == 2 ? 12 : 6;       // plane words per weight dword
  static constexpr int SLOT = 4 * PWD + 4;             // words per chunk slot (52 / 28)
};

// Stage chunks [c0, c0 + SC) of every A row as planes; meta[(m*4+gi)*SC + slot] =
// {2^(e-22), sum a} for scale group gi of the slot.  A group whose largest |a| is
// not finite gets a NaN step, so the rows it meets come out NaN.
template <int BITS, int AT, int G>
__device__ __forceinline__ void stage_planes(const GemvArgs& g, uint32_t* planes, f32x2* meta, int c0,
                                             int SC) {
  using L = IpLayout<BITS>;
  constexpr int WPC = 128 / BITS;
  constexpr int NB = 8;  // float4 pieces per thread whose loads are issued together
  const int per_row = SC * (WPC / 4);  // float4 pieces per A row in the slice
  const int total = (int)g.M * per_row;
  const int K = (int)g.K;
  constexpr int gw = G / 4;  // threads per scale group (4, 8 or 16: aligned groups of lanes)
  auto load = [&](int idx, float (&v)[4]) {
    v[0] = v[1] = v[2] = v[3] = 0.0f;
    if (idx >= total) return;
    const int m = idx / per_row;
    const int rem = idx - m * per_row;
    const int k = (c0 * WPC) + 4 * rem;
    const int64_t base = (int64_t)m * K + k;
    if (g.a_vec && k + 3 < K) {
      if constexpr (AT == QMM_F32) {
        const f32x4 x = *(const f32x4*)((const float*)g.A + base);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      } else {
        const uint2 u = *(const uint2*)((const uint16_t*)g.A + base);
        const uint32_t w[2] = {u.x, u.y};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if constexpr (AT == QMM_F16) {
            v[2 * e] = f16_to_f32((uint16_t)(w[e] & 0xffffu));
            v[2 * e + 1] = f16_to_f32((uint16_t)(w[e] >> 16));
          } else {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (k + e < K) ? load_elem<AT>(g.A, base + e) : 0.0f;
    }
  };
  // NB rounds of pieces at a time: all loads first (one memory latency per batch),
  // then the conversion; every lane takes part in the group butterflies
  for (int base_idx = 0; base_idx < total; base_idx += NB * (int)blockDim.x) {
    float vb[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j) load(base_idx + j * (int)blockDim.x + (int)threadIdx.x, vb[j]);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (base_idx + j * (int)blockDim.x >= total) break;  // uniform over the work-group
      const int idx = base_idx + j * (int)blockDim.x + (int)threadIdx.x;
      const bool ok = idx < total;
      const float* v = vb[j];
      const int m = ok ? idx / per_row : 0;
      const int rem = idx - m * per_row;
      const int slot = rem / (WPC / 4);
      const int j4 = rem - slot * (WPC / 4);  // float4 piece inside the chunk
      // group maximum and group sum over the gw threads of the group (DPP exchanges)
      float mx = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
      float sm = ((v[0] + v[1]) + v[2]) + v[3];
      mx = fmaxf(mx, dpp_f<kDppXor1>(mx));
      sm += dpp_f<kDppXor1>(sm);
      mx = fmaxf(mx, dpp_f<kDppXor2>(mx));
      sm += dpp_f<kDppXor2>(sm);
      if constexpr (gw >= 8) {
        mx = fmaxf(mx, dpp_f<kDppHalfMirror>(mx));
        sm += dpp_f<kDppHalfMirror>(sm);
      }
      if constexpr (gw >= 16) {
        mx = fmaxf(mx, dpp_f<kDppMirror>(mx));
        sm += dpp_f<kDppMirror>(sm);
      }
      int e = 0;
      (void)frexpf(mx, &e);  // mx < 2^e (mx = 0 gives e = 0)
      if (!ok) continue;
      uint32_t u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = (uint32_t)(int)rintf(ldexpf(v[q], 22 - e));
      uint32_t* slot_w = planes + (m * SC + slot) * L::SLOT;
      if constexpr (BITS == 2) {
        // elements j0..j0+3 of a 16-code dword: j0, j0+2 even (nibbles j0/2, j0/2+1 of
        // the E words), j0+1, j0+3 odd (same nibbles of the O words).  Digit p of two
        // values goes to one byte: the low nibbles of bytes 0-2 of a value are its
        // digits 0, 2, 4, the high nibbles its digits 1, 3, 5 (24-bit two's complement).
        const int d = (4 * j4) >> 4;
        const int qb = ((4 * j4) & 15) >> 2;  // byte of each plane word
        uint8_t* wb = (uint8_t*)(slot_w + d * L::PWD) + qb;
        const uint32_t ee = (u[0] & 0x0F0F0Fu) | ((u[2] << 4) & 0xF0F0F0u);  // E digits 0, 2, 4
        const uint32_t eo = ((u[0] >> 4) & 0x0F0F0Fu) | (u[2] & 0xF0F0F0u);  // E digits 1, 3, 5
        const uint32_t oe = (u[1] & 0x0F0F0Fu) | ((u[3] << 4) & 0xF0F0F0u);
        const uint32_t oo = ((u[1] >> 4) & 0x0F0F0Fu) | (u[3] & 0xF0F0F0u);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          wb[(2 * (2 * k)) * 4] = (uint8_t)(ee >> (8 * k));
          wb[(2 * (2 * k + 1)) * 4] = (uint8_t)(eo >> (8 * k));
          wb[(2 * (2 * k) + 1) * 4] = (uint8_t)(oe >> (8 * k));
          wb[(2 * (2 * k + 1) + 1) * 4] = (uint8_t)(oo >> (8 * k));
        }
      } else {
        // elements j0..j0+3 of an 8-code dword are nibbles j0..j0+3 of each plane word
        // (digits of a + 2^23): pair the values, then join the two pairs' bytes
        const int d = (4 * j4) >> 3;
        const int qh = ((4 * j4) & 7) >> 2;  // half-word of each plane word
        uint16_t* wh = (uint16_t*)(slot_w + d * L::PWD) + qh;
#pragma unroll
        for (int q = 0; q < 4; ++q) u[q] += 1u << 23;
        const uint32_t x01 = (u[0] & 0x0F0F0Fu) | ((u[1] << 4) & 0xF0F0F0u);  // digits 0, 2, 4
        const uint32_t y01 = ((u[0] >> 4) & 0x0F0F0Fu) | (u[1] & 0xF0F0F0u);  // digits 1, 3, 5
        const uint32_t x23 = (u[2] & 0x0F0F0Fu) | ((u[3] << 4) & 0xF0F0F0u);
        const uint32_t y23 = ((u[2] >> 4) & 0x0F0F0Fu) | (u[3] & 0xF0F0F0u);
        // byte k of a pair word + byte k of the other pair word = the plane's half-word
        const uint32_t p02 = __builtin_amdgcn_perm(x23, x01, 0x05010400u);  // digits 0 | 2
        const uint32_t p13 = __builtin_amdgcn_perm(y23, y01, 0x05010400u);  // digits 1 | 3
        const uint32_t p45 = __builtin_amdgcn_perm(y23, y01, 0x06020000u) & 0xffff0000u;
        const uint32_t p4 = __builtin_amdgcn_perm(x23, x01, 0x00000602u) & 0xffffu;
        wh[0 * 2] = (uint16_t)p02;
        wh[2 * 2] = (uint16_t)(p02 >> 16);
        wh[1 * 2] = (uint16_t)p13;
        wh[3 * 2] = (uint16_t)(p13 >> 16);
        wh[4 * 2] = (uint16_t)p4;
        wh[5 * 2] = (uint16_t)(p45 >> 16);
      }
      if ((j4 % gw) == 0) {
        const int gi = j4 / gw;
        f32x2 mt;
        mt.x = mx <= 3.402823466e38f ? ldexpf(1.0f, e - 22) : __builtin_nanf("");
        mt.y = sm;
        meta[(m * 4 + gi) * SC + slot] = mt;
      }
    }
  }
}

// General form (A staged one K-slice at a time inside the item loop, row sums
// written out whenever the LDS buffer fills); qmm_gemv_stream.h holds the
// streaming form for rows whose activations fit in LDS whole.
// DPG: weight dwords per scale group inside a chunk (4 = the chunk lies in one block).
template <int BITS, int AT, int MT, int R, int DPG, int ZK>
__global__ __launch_bounds__(kGemvThreads) void gemv_ip_kernel(GemvArgs g) {
  using L = IpLayout<BITS>;
  constexpr int WPC = 128 / BITS;
  constexpr int G = DPG * L::WPD;  // codes per scale group inside a chunk
  constexpr int NS = 4 / DPG;      // scale groups per chunk
  constexpr int NWAVES = kGemvThreads / 64;
  extern __shared__ float lds[];
  const int SC = g.slice_chunks;
  uint32_t* planes = (uint32_t*)lds;
  f32x2* meta = (f32x2*)(planes + MT * SC * L::SLOT);
  float* out_lds = (float*)(meta + MT * 4 * SC);
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
  const int tiles_lo = ntiles / gridDim.x, extra = ntiles % gridDim.x;
  const int t_begin = blockIdx.x * tiles_lo + (blockIdx.x < extra ? blockIdx.x : extra);
  const int t_end = t_begin + tiles_lo + (blockIdx.x < extra ? 1 : 0);
  if (t_begin >= t_end) return;
  const int nchunks = (int)g.nchunks;
  const int nslices = (nchunks + SC - 1) / SC;
  const int iters = SC >> lpr_log2;
  const int nblk = (int)g.nblk;
  const int blog = g.block_log2;
  const int64_t row_bytes = g.row_bytes;
  const float zconst = g.zp_kind == QMM_ZP_UNIFORM ? g.uniform_zp : (float)(1 << (BITS - 1));
  const int zrow_bytes = (int)g.zp_row_bytes;
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
  ItemPos fpos{t_begin, 0, 0};
  int fchunk = lp;
  const uint8_t* fw[R];
  const _Float16* fsa[R];
  const uint8_t* fzp[R];
  const _Float16* fzh[R];
  auto set_bases = [&](int tl) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int row = tl * rows_per_tile + wave * rows_per_wave + r * SUBS + sub;
      row = (tl < t_end && row < N) ? row : N - 1;
      fw[r] = g.W + (int64_t)row * row_bytes;
      fsa[r] = (const _Float16*)g.scales + (int64_t)row * nblk;
      if constexpr (ZK == 1) fzp[r] = (const uint8_t*)g.zp + (int64_t)row * zrow_bytes;
      if constexpr (ZK == 2) fzh[r] = (const _Float16*)g.zp + (int64_t)row * nblk;
    }
  };
  set_bases(t_begin);
  auto fetch_next = [&](IpBuf<R, NS>& b) {
    const int cc = (fpos.tile < t_end && fchunk < nchunks) ? fchunk : nchunks - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      b.w[r] = *(const uint4*)(fw[r] + cc * 16);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int bidx = (cc * WPC + i * G) >> blog;
        b.s[r][i] = fsa[r][bidx];
        if constexpr (ZK == 1) {
          const int bit = bidx * BITS;
          b.z[r][i] = fzp[r][bit >> 3];
          b.zsh[r][i] = bit & 7;
        } else if constexpr (ZK == 2) {
          b.zh[r][i] = fzh[r][bidx];
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

  ItemPos cur{t_begin, 0, 0};
  bool staged = false;
  int flush_from = t_begin;
  // items of every lane of this work-group; `live` is uniform over the work-group
  const int total_items = (t_end - t_begin) * nslices * iters;

  auto step = [&](IpBuf<R, NS>& cbuf, IpBuf<R, NS>& nxt, bool live) {
    if (live && cur.it == 0 && (nslices > 1 || !staged)) {
      __syncthreads();
      stage_planes<BITS, AT, G>(g, planes, meta, cur.s * SC, SC);
      __syncthreads();
      staged = true;
    }
    fetch_next(nxt);

    // computed for every lane (no branch around it, so the register sets of the
    // ring stay in flight on every path); chunks past the row end are discarded
    const int slot = cur.it * LPR + lp;
    const bool valid = live && cur.s * SC + slot < nchunks;
    {
      const uint32_t* pb = planes + slot * L::SLOT;
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
            const f32x2 mt = meta[(mm * 4 + gi) * SC + slot];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              int s5 = S[r][m][5];
              if constexpr (BITS == 4) s5 -= 8 * Sq[r];  // remove the 2^23 bias of a_int
              // both halves stay below 2^24 in magnitude, so P is rounded once
              const int lo = S[r][m][0] + (S[r][m][1] << 4) + (S[r][m][2] << 8);
              const int hi = S[r][m][3] + (S[r][m][4] << 4) + s5 * 256;
              const float P = fmaf((float)hi, 4096.0f, (float)lo);
              const float scv = (float)cbuf.s[r][gi];
              float z;
              if constexpr (ZK == 1) z = (float)((cbuf.z[r][gi] >> cbuf.zsh[r][gi]) & ((1u << BITS) - 1u));
              else if constexpr (ZK == 2) z = (float)cbuf.zh[r][gi];
              else z = zconst;
              // same expression for every zero-point kind, so a uniform scalar and
              // a tensor holding that value give the same bits
              const float nv = fmaf(scv, fmaf(-z, mt.y, P * mt.x), acc[r][m]);
              acc[r][m] = valid ? nv : acc[r][m];
            }
          }
        }
      }
    }

    if (live && cur.s == nslices - 1 && cur.it == iters - 1) {
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
    }
    advance(cur);
  };

  // ring of kIpDepth register sets; the loop body is unrolled so that set indices
  // are constants and the sets rotate without copies
  IpBuf<R, NS> buf[kIpDepth];
#pragma unroll
  for (int i = 0; i < kIpDepth - 1; ++i) fetch_next(buf[i]);
  // whole rounds of kIpDepth steps; steps past the last item only issue clamped
  // loads and discard their results
  for (int base = 0; base < total_items; base += kIpDepth) {
#pragma unroll
    for (int i = 0; i < kIpDepth; ++i) step(buf[i], buf[(i + kIpDepth - 1) % kIpDepth], base + i < total_items);
  }
}

}  // namespace qmm
