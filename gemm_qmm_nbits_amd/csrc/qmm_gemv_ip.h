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
// One dominant activation per group is taken out of the planes: when the largest
// magnitude of a group is at least 32 times the second largest (an activation
// outlier), that value is staged as zero and left out of the group sum, the exponent
// e comes from the second largest, and its own term a_o * (q_o - zp) is added in fp32
// to P * 2^(e-22).  The fixed-point error of the other values is then bounded by
// 2^-23 of the second largest magnitude instead of the outlier's, and the zero-point
// fold never subtracts two outlier-sized terms.
//
// The work decomposition (lanes per row, lane -> chunk map, per-lane chunk order,
// fixed xor butterfly, tiles, prefetch ring, LDS output buffer) is that of the
// fp32 kernel in qmm_gemv_impl.h, so the summation order again depends only on
// (K, block, bits).
#pragma once
#include "qmm_gemv_impl.h"

#include <type_traits>

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

// Nibble planes of eight 24-bit values: word p (p = 0..5) holds digit p (bits 4p..4p+3)
// of value i in nibble i.  x holds byte k of values 0, 2, 4, 6 and y of values 1, 3,
// 5, 7 (built by byte_gather), so the even digit 2k of value 2b is the low nibble
// of byte b of x_k.
__device__ __forceinline__ void byte_gather(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t (&x)[3]) {
  // x[k] = [byte k of a, byte k of b, byte k of c, byte k of d] (a in byte 0)
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  x[0] = __builtin_amdgcn_perm(cd, ab, 0x05040100u);
  x[1] = __builtin_amdgcn_perm(cd, ab, 0x07060302u);
  x[2] = __builtin_amdgcn_perm(b, a, 0x0c0c0602u) | __builtin_amdgcn_perm(d, c, 0x06020c0cu);
}
__device__ __forceinline__ void nibble_planes(const uint32_t (&x)[3], const uint32_t (&y)[3], uint32_t (&w)[6]) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    w[2 * k] = (x[k] & 0x0F0F0F0Fu) | ((y[k] << 4) & 0xF0F0F0F0u);
    w[2 * k + 1] = ((x[k] >> 4) & 0x0F0F0F0Fu) | (y[k] & 0xF0F0F0F0u);
  }
}

// Stage chunks [c0, c0 + SC) of every A row as planes; meta[(m*4+gi)*SC + slot] =
// {2^(e-22), sum a, a_o, index of a_o in the group (as bits)} for scale group gi of
// the slot, a_o = 0 when no value is taken out.  A group whose largest |a| is not
// finite, or that holds a NaN, gets a NaN step, so the rows it meets come out NaN.
//
// Each thread converts 16 consecutive activations (one 2-bit weight dword, two
// 4-bit ones): the 12 plane words they fill are contiguous in the slot, so they
// are built in registers and written as three 16-byte stores.  A scale group of G
// codes spans G / 16 neighbouring lanes; its maximum and sum are DPP butterflies.
// `issued` runs once (there is at least one piece), right after the loads of the
// first batch are issued: a caller
// that starts its own loads there (the first weights of its stream) lets them travel
// while the activations are converted, and waiting for the activations, which are
// issued first, does not wait for them (vector loads complete in order).
// AVEC: rows of A allow 4-element vector loads.  Loads are branch-free, so all loads
// of a batch are in flight together.  BUF (A below 2 GiB): raw buffer loads, with an
// offset past the buffer's range for an element past the row or a piece past the
// last, which returns 0 and fetches nothing.  Otherwise global loads, whose address
// is replaced by the first element and whose value by a select.
// Position of this lane's 16-value piece inside its scale group of GW pieces: the
// pieces of a group are staged by GW consecutive lanes (batches start at multiples of
// the work-group size).
template <int GW>
__device__ __forceinline__ int piece_of_lane() {
  return (int)(threadIdx.x & (unsigned)(GW - 1));
}

// The product of a value taken out of a scale group with its code: the code sits in
// dword gi * DPG + id / (32 / BITS) of the chunk, field id % (32 / BITS).
template <int BITS, int DPG>
__device__ __forceinline__ float outlier_code(const uint4& w, int gi, uint32_t id) {
  constexpr uint32_t WPD = 32 / BITS;
  const uint32_t di = (uint32_t)(gi * DPG) + id / WPD;
  const uint32_t x = di == 0 ? w.x : di == 1 ? w.y : di == 2 ? w.z : w.w;
  return (float)((x >> ((id % WPD) * BITS)) & ((1u << BITS) - 1u));
}

template <int BITS, int AT, int G, int MT, bool AVEC, bool BUF, bool MX, typename Issued>
__device__ __forceinline__ void stage_planes_impl(const GemvArgs& g, uint32_t* planes, f32x4* meta,
                                                  uint32_t* trash, int c0, int SC, Issued&& issued) {
  using L = IpLayout<BITS>;
  constexpr int WPC = 128 / BITS;
  constexpr int PPC = WPC / 16;  // 16-value pieces per chunk (4 or 2)
  constexpr int NB = 2;          // pieces per thread whose loads are issued together
  const int per_row = SC * PPC;
  const int total = (int)g.M * per_row;
  const int K = (int)g.K;
  constexpr int gw = G / 16;  // threads per scale group (1, 2 or 4: aligned groups of lanes)
  static_assert(gw == 1 || gw == 2 || gw == 4, "scale group of 16, 32 or 64 codes");
  constexpr uint32_t ES = AT == QMM_F32 ? 4 : 2;
  constexpr uint32_t kOut = 0x80000000u;  // past the buffer's range (< 2^31 bytes)
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(g.A), (short)0, BUF ? (int)((uint32_t)g.M * (uint32_t)K * ES) : 0, 0x00020000);
  const uint32_t trash_word = (uint32_t)(trash - planes);
  const uint32_t meta_word = (uint32_t)((uint32_t*)meta - planes);
  auto to_f32 = [](uint32_t w, int half) -> float {
    const uint32_t h = half ? w >> 16 : w & 0xffffu;
    if constexpr (AT == QMM_F16) return f16_to_f32((uint16_t)h);
    else return __uint_as_float(h << 16);
  };
  // row m of piece idx (< MT rows) and its first piece, by compares: no division
  auto row_of = [&](uint32_t idx, uint32_t& m, uint32_t& first) {
    m = 0;
    first = 0;
#pragma unroll
    for (int r = 1; r < MT; ++r) {
      const bool ge = idx >= (uint32_t)(r * per_row);
      m += ge ? 1u : 0u;
      first = ge ? (uint32_t)(r * per_row) : first;
    }
  };
  auto load = [&](int idx, float (&v)[16]) {
    const bool okp = idx < total;
    uint32_t m, first;
    row_of(okp ? (uint32_t)idx : 0u, m, first);
    const int k = c0 * WPC + 16 * (int)((okp ? (uint32_t)idx : 0u) - first);
    const int64_t base = (int64_t)m * K + k;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kq = k + 4 * q;
      if constexpr (BUF) {
        if constexpr (AVEC) {
          const uint32_t off = okp && kq < K ? (uint32_t)(base + 4 * q) * ES : kOut;
          if constexpr (AT == QMM_F32) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(rA, (int)off, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = __uint_as_float(t[e]);
          } else {
            const auto t = __builtin_amdgcn_raw_buffer_load_b64(rA, (int)off, 0, 0);
            v[4 * q] = to_f32(t[0], 0);
            v[4 * q + 1] = to_f32(t[0], 1);
            v[4 * q + 2] = to_f32(t[1], 0);
            v[4 * q + 3] = to_f32(t[1], 1);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t off = okp && kq + e < K ? (uint32_t)(base + 4 * q + e) * ES : kOut;
            if constexpr (AT == QMM_F32)
              v[4 * q + e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rA, (int)off, 0, 0));
            else
              v[4 * q + e] = to_f32(__builtin_amdgcn_raw_buffer_load_b16(rA, (int)off, 0, 0), 0);
          }
        }
      } else if constexpr (AVEC) {
        const bool ok = okp && kq < K;  // K % 4 == 0: kq < K means all four are in the row
        const int64_t off = ok ? base + 4 * q : 0;
        float x[4];
        if constexpr (AT == QMM_F32) {
          const f32x4 t = *(const f32x4*)((const float*)g.A + off);
          x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
        } else {
          const uint2 u = *(const uint2*)((const uint16_t*)g.A + off);
          const uint32_t w[2] = {u.x, u.y};
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            if constexpr (AT == QMM_F16) {
              x[2 * e] = f16_to_f32((uint16_t)(w[e] & 0xffffu));
              x[2 * e + 1] = f16_to_f32((uint16_t)(w[e] >> 16));
            } else {
              x[2 * e] = __uint_as_float(w[e] << 16);
              x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = ok ? x[e] : 0.0f;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = okp && kq + e < K;
          const float x = load_elem<AT>(g.A, ok ? base + 4 * q + e : 0);
          v[4 * q + e] = ok ? x : 0.0f;
        }
      }
    }
  };
  // NB pieces at a time: all loads first (one memory latency per batch), then the
  // conversion; every lane takes part in the group butterflies
  // the first batch is peeled so that the caller's loads are issued on every path
  // (a conditional issue would make the compiler wait for them with the batch)
  // first piece of this wave's lanes, as a scalar: a wave with no piece in a batch
  // skips it (a branch on a scalar, so no lane of the wave waits at the join)
  const int wave_base = __builtin_amdgcn_readfirstlane((int)(threadIdx.x & ~63u));
  auto batch = [&](int base_idx, auto first) {
    float vb[NB][16];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (base_idx + j * (int)blockDim.x + wave_base < total)
        load(base_idx + j * (int)blockDim.x + (int)threadIdx.x, vb[j]);
    if constexpr (decltype(first)::value) {
      __builtin_amdgcn_sched_barrier(0);  // keep the caller's loads behind these
      issued();
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (base_idx + j * (int)blockDim.x + wave_base >= total) break;  // uniform over the wave
      const int idx = base_idx + j * (int)blockDim.x + (int)threadIdx.x;
      const bool ok = idx < total;
      float* v = vb[j];
      // piece index = (m * SC + slot) * PPC + piece: chunk slot cs = m * SC + slot, and
      // the 16-value piece inside the chunk (24-bit products: no 64-bit arithmetic)
      const uint32_t uidx = ok ? (uint32_t)idx : 0u;
      const uint32_t cs = uidx / (uint32_t)PPC;
      const uint32_t piece = uidx % (uint32_t)PPC;
      uint32_t m, first;
      row_of(uidx, m, first);
      // largest magnitude m1 (its index in the group and its value), second largest m2
      float m1 = 0.0f, m2 = 0.0f, vo = 0.0f;
      uint32_t io = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float a = fabsf(v[q]);
        const bool top = a > m1;
        m2 = top ? m1 : fmaxf(m2, a);
        io = top ? (uint32_t)q : io;
        vo = top ? v[q] : vo;
        m1 = top ? a : m1;
      }
      io += (uint32_t)(piece_of_lane<gw>() * 16);
      // combine with the partner lane's record: the larger value wins (ties to the lower
      // index), the loser's maximum competes for second place; partners agree bitwise
      auto combine = [&](float om1, uint32_t oio, float om2, float ovo) {
        const bool take = om1 > m1 || (om1 == m1 && oio < io);
        m2 = take ? fmaxf(om2, m1) : fmaxf(m2, om1);
        io = take ? oio : io;
        vo = take ? ovo : vo;
        m1 = take ? om1 : m1;
      };
      if constexpr (gw >= 2) {
        const float om1 = dpp_f<kDppXor1>(m1), om2 = dpp_f<kDppXor1>(m2), ovo = dpp_f<kDppXor1>(vo);
        const uint32_t oio = (uint32_t)__float_as_int(dpp_f<kDppXor1>(__int_as_float((int)io)));
        combine(om1, oio, om2, ovo);
      }
      if constexpr (gw >= 4) {
        const float om1 = dpp_f<kDppXor2>(m1), om2 = dpp_f<kDppXor2>(m2), ovo = dpp_f<kDppXor2>(vo);
        const uint32_t oio = (uint32_t)__float_as_int(dpp_f<kDppXor2>(__int_as_float((int)io)));
        combine(om1, oio, om2, ovo);
      }
      // a dominant value is taken out of the planes and of the group sum (finite,
      // nonzero, at least 32 times every other magnitude); its product is added apart
      const bool excl = m1 <= 3.402823466e38f && m1 > 0.0f && m1 >= 32.0f * m2;
      const uint32_t own = excl && (io >> 4) == (uint32_t)piece_of_lane<gw>() ? (io & 15u) : 16u;
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = (uint32_t)q == own ? 0.0f : v[q];
      float sm = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) sm += ((v[4 * q] + v[4 * q + 1]) + v[4 * q + 2]) + v[4 * q + 3];
      if constexpr (gw >= 2) sm += dpp_f<kDppXor1>(sm);
      if constexpr (gw >= 4) sm += dpp_f<kDppXor2>(sm);
      const bool finite = m1 <= 3.402823466e38f && sm == sm;
      const float mx = excl ? m2 : m1;
      int e = 0;
      (void)frexpf(mx, &e);  // mx < 2^e (mx = 0 gives e = 0)
      uint32_t u[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) u[q] = (uint32_t)(int)rintf(ldexpf(v[q], 22 - e));
      uint32_t w[12];
      if constexpr (MX) {
        // matrix-core operand (2-bit codes, one group per chunk, one A row): chunk cs is
        // chunk j = cs % 4 of pair u = cs / 4; digit p of the piece's 16 values goes as 16
        // e4m3 bytes (the even values first) to operand region 2 * (j / 2) + piece / 2 of
        // the pair, lane slot 16 * (2 * (j % 2) + piece % 2) + row(p), with row(p) =
        // 8 * (j % 2) + 4 * (p / 3) + p % 3 (the six planes as two triples)
        static_assert(BITS == 2 && G == 64 && MT == 1, "matrix-core staging: 2-bit, one group per chunk, M = 1");
        const uint32_t j = cs & 3u;
        const uint32_t base = __umul24(cs >> 2, 1024u) + (2u * (j >> 1) + (piece >> 1)) * 256u +
                              (16u * (2u * (j & 1u) + (piece & 1u))) * 4u;
#pragma unroll
        for (int p = 0; p < 6; ++p) {
          auto digit = [&](uint32_t x) -> float {
            return p < 5 ? (float)(int)((x >> (4 * p)) & 15u) : (float)(((int)(x << 8)) >> 28);
          };
          uint32_t pk[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int i0 = k < 2 ? 8 * k : 8 * (k - 2) + 1;
            int x = __builtin_amdgcn_cvt_pk_fp8_f32(digit(u[i0]), digit(u[i0 + 2]), 0, false);
            x = __builtin_amdgcn_cvt_pk_fp8_f32(digit(u[i0 + 4]), digit(u[i0 + 6]), x, true);
            pk[k] = (uint32_t)x;
          }
          const uint32_t row = (j & 1u) * 8u + 4u * (uint32_t)(p / 3) + (uint32_t)(p % 3);
          *(uint4*)(planes + (ok ? base + row * 4u : trash_word)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
      } else if constexpr (BITS == 2) {
        // even values (nibble i of the E planes = value 2i), then odd values (O planes)
        uint32_t ex[3], ey[3], ox[3], oy[3], ew[6], ow[6];
        byte_gather(u[0], u[4], u[8], u[12], ex);
        byte_gather(u[2], u[6], u[10], u[14], ey);
        byte_gather(u[1], u[5], u[9], u[13], ox);
        byte_gather(u[3], u[7], u[11], u[15], oy);
        nibble_planes(ex, ey, ew);
        nibble_planes(ox, oy, ow);
#pragma unroll
        for (int p = 0; p < 6; ++p) {
          w[2 * p] = ew[p];
          w[2 * p + 1] = ow[p];
        }
      } else {
        // digits of a + 2^23; values 0..7 fill the six words of the first dword,
        // values 8..15 those of the second
#pragma unroll
        for (int q = 0; q < 16; ++q) u[q] += 1u << 23;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t x[3], y[3], pw[6];
          byte_gather(u[8 * h], u[8 * h + 2], u[8 * h + 4], u[8 * h + 6], x);
          byte_gather(u[8 * h + 1], u[8 * h + 3], u[8 * h + 5], u[8 * h + 7], y);
          nibble_planes(x, y, pw);
#pragma unroll
          for (int p = 0; p < 6; ++p) w[6 * h + p] = pw[p];
        }
      }
      // lanes without a piece (and the meta record of all but the group's first lane)
      // write to the trash line instead of branching around the stores
      // (32-bit word offsets from the planes, so the choice is one select)
      if constexpr (!MX) {
        const uint32_t pw = ok ? __umul24(cs, (uint32_t)L::SLOT) + __umul24(piece, 12u) : trash_word;
        uint4* dst = (uint4*)(planes + pw);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        dst[2] = make_uint4(w[8], w[9], w[10], w[11]);
      }
      f32x4 mt;
      mt.x = finite ? ldexpf(1.0f, e - 22) : __builtin_nanf("");
      mt.y = sm;
      mt.z = excl ? vo : 0.0f;
      mt.w = __uint_as_float(excl ? io : 0u);
      // record (m * 4 + gi) * SC + slot = cs + (3 m + gi) * SC, by selects
      const uint32_t gi = piece / gw;
      const uint32_t usc = (uint32_t)SC;
      const uint32_t gsc = gi == 0 ? 0u : gi == 1 ? usc : gi == 2 ? 2u * usc : 3u * usc;
      uint32_t m3 = 0;
#pragma unroll
      for (int r = 1; r < MT; ++r) m3 += m >= (uint32_t)r ? 3u * usc : 0u;
      const uint32_t mw = ok && (piece % gw) == 0 ? meta_word + 4u * (cs + m3 + gsc) : trash_word;
      *(f32x4*)(planes + mw) = mt;
    }
  };
  batch(0, std::true_type{});
  for (int base_idx = NB * (int)blockDim.x; base_idx < total; base_idx += NB * (int)blockDim.x)
    batch(base_idx, std::false_type{});
}

// trash: 64 bytes of LDS (16-byte aligned) that nothing reads.  BUF requires
// M * K * element size < 2^31 - 64 (the streaming kernel's A fits in LDS).
template <int BITS, int AT, int G, int MT, bool BUF, typename Issued>
__device__ __forceinline__ void stage_planes(const GemvArgs& g, uint32_t* planes, f32x4* meta,
                                             uint32_t* trash, int c0, int SC, Issued&& issued) {
  if (g.a_vec)
    stage_planes_impl<BITS, AT, G, MT, true, BUF, false>(g, planes, meta, trash, c0, SC, issued);
  else
    stage_planes_impl<BITS, AT, G, MT, false, BUF, false>(g, planes, meta, trash, c0, SC, issued);
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
      stage_planes<BITS, AT, G, MT, false>(g, planes, meta, trash, cur.s * SC, SC, [] {});
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
            const f32x4 mt = meta[(mm * 4 + gi) * SC + slot];
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
              float t = P * mt.x;
              // a value taken out of the planes: a_o * (q_o - zp), q_o - zp exact
              if (mt.z != 0.0f)
                t = fmaf(mt.z, outlier_code<BITS, DPG>(cbuf.w[r], gi, __float_as_uint(mt.w)) - z, t);
              // same expression for every zero-point kind, so a uniform scalar and
              // a tensor holding that value give the same bits
              const float nv = fmaf(scv, fmaf(-z, mt.y, t), acc[r][m]);
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
