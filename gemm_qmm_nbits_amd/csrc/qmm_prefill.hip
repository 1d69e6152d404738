// Prefill (large M) path of MatMulNBits on the fp16 matrix cores
// ([P1] hip-ep PR 1318, "What", commit 1: the prefill tiles re-read A once per
// N block, so A is cast to fp16 once and fp32 C is written from the epilogue;
// "Performance"/Qwen study: prefill is compute bound).
//
// C[M][N] = A16 . W16^T (+ bias), with A16 = fp16(A) (cast once into the caller's
// workspace by launch_cast_to_f16) and W16 = fp16(fp32(fp32(q - zp) * s)), the
// round-to-nearest fp16 of the exact dequantized weight, built tile by tile in LDS.
// Products are accumulated in fp32 by v_mfma_f32_32x32x16_f16 in increasing k order
// (64 codes per stage), whatever the tile shape.
//
// Work-group: 256 threads (4 waves), output tile BM x BN = 256 x 256, each wave a
// 128 x 128 quarter held as 4 x 4 MFMA blocks of 32 x 32 (fp32 accumulators).  Each
// stage stages A[256][64] (fp16) and W16[256][64] in LDS (rows padded to 72 halves
// so the 16-byte operand reads of a wave hit distinct banks), double buffered with
// one barrier per stage: the next stage's global loads are issued before the MFMAs
// of the current one and written to the other buffer after them.
//
// MFMA operand layout (32x32x16 f16): lane l holds row (or column) l % 32 and the 8
// consecutive k at 8 * (l / 32); accumulator v of lane l is row 8*(v/4) + 4*(l/32)
// + v%4, column l % 32.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int LDA = BK + 8;  // padded LDS row (halves)
constexpr int NT = 256;      // threads

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return (uint32_t)f32_to_f16(a) | ((uint32_t)f32_to_f16(b) << 16);
}

// Raw codes, scales and zero points of 64 codes of weight row n starting at k0.
template <int BITS>
struct BStage {
  uint32_t raw[2 * BITS];  // 64 codes: 2-bit -> 4 dwords, 4-bit -> 8 dwords
  float sc[4];             // per 16 codes (a block holds >= 16 codes)
  float zz[4];
};

template <int BITS, int ZK>
__device__ __forceinline__ void load_b(const PrefillArgs& p, int n, int k0, BStage<BITS>& b) {
  const bool row_ok = n < p.N;
  const int kpad = (int)(p.nblk * p.block);
  const uint8_t* row = p.W + (int64_t)(row_ok ? n : 0) * p.row_bytes;
  if (row_ok && k0 + BK <= kpad && p.w_vec) {
    const uint4* src = (const uint4*)(row + ((k0 * BITS) >> 3));
#pragma unroll
    for (int q = 0; q < BITS / 2; ++q) {
      const uint4 v = src[q];
      b.raw[4 * q + 0] = v.x;
      b.raw[4 * q + 1] = v.y;
      b.raw[4 * q + 2] = v.z;
      b.raw[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int d = 0; d < 2 * BITS; ++d) {
      uint32_t x = 0;
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        const int kb = k0 + (d * 4 + by) * (8 / BITS);  // first code of this byte
        if (row_ok && kb < kpad) x |= (uint32_t)row[(kb * BITS) >> 3] << (8 * by);
      }
      b.raw[d] = x;
    }
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    int blk = (k0 + 16 * h) >> p.block_log2;
    if (blk >= p.nblk) blk = (int)p.nblk - 1;
    const int64_t si = (int64_t)(row_ok ? n : 0) * p.nblk + blk;
    b.sc[h] = f16_to_f32(p.scales[si]);
    if constexpr (ZK == 1) {
      const uint8_t* zr = (const uint8_t*)p.zp + (int64_t)(row_ok ? n : 0) * p.zp_row_bytes;
      const int bit = blk * BITS;
      b.zz[h] = (float)((zr[bit >> 3] >> (bit & 7)) & ((1u << BITS) - 1u));
    } else if constexpr (ZK == 2) {
      b.zz[h] = f16_to_f32(((const uint16_t*)p.zp)[si]);
    } else {
      b.zz[h] = p.zconst;
    }
  }
}

// Dequantize 64 codes to fp16 in k order and store them as one padded LDS row.
template <int BITS>
__device__ __forceinline__ void store_b(const BStage<BITS>& b, uint16_t* dst_row) {
  uint32_t o[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int k = 2 * j;  // codes k, k+1 of the stage
    const int h = k >> 4;
    const uint32_t q0 = (b.raw[(k * BITS) >> 5] >> ((k * BITS) & 31)) & ((1u << BITS) - 1u);
    const uint32_t q1 = (b.raw[((k + 1) * BITS) >> 5] >> (((k + 1) * BITS) & 31)) & ((1u << BITS) - 1u);
    const float w0 = __fmul_rn(__fsub_rn((float)q0, b.zz[h]), b.sc[h]);
    const float w1 = __fmul_rn(__fsub_rn((float)q1, b.zz[h]), b.sc[h]);
    o[j] = pack_h2(w0, w1);
  }
  uint4* dst = (uint4*)dst_row;
#pragma unroll
  for (int q = 0; q < 8; ++q) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

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

template <int BITS, int ZK, int CT>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_h[];
  uint16_t* As = smem_h;                  // [2][BM * LDA]
  uint16_t* Bs = smem_h + 2 * BM * LDA;   // [2][BN * LDA]

  // tile order: the M tiles of one N tile run on one XCD (work-groups are dealt
  // round-robin over 8 XCDs), so the packed weights of that N tile are read into
  // one L2
  const int i = blockIdx.x;
  const int x = i & 7, j = i >> 3;
  const int nt = (j / p.mtiles) * 8 + x;
  const int mt = j % p.mtiles;
  if (nt >= p.ntiles) return;
  const int m0 = mt * BM, n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, 128 x 128 each
  const int K = (int)p.K;
  const int nsteps = (K + BK - 1) / BK;

  // A stage: thread -> row m0 + tid, 64 halves (8 x 16 bytes)
  const int a_row = m0 + tid;
  const bool a_ok = a_row < p.M;
  const uint16_t* arow = p.A16 + (int64_t)(a_ok ? a_row : 0) * K;
  auto load_a = [&](int k0, uint4 (&v)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int k = k0 + 8 * q;
      if (a_ok && p.a_vec && k + 8 <= K) {
        v[q] = *(const uint4*)(arow + k);
      } else {
        uint32_t t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (a_ok && k + 2 * e < K) ? arow[k + 2 * e] : 0u;
          const uint32_t hi = (a_ok && k + 2 * e + 1 < K) ? arow[k + 2 * e + 1] : 0u;
          t[e] = lo | (hi << 16);
        }
        v[q] = make_uint4(t[0], t[1], t[2], t[3]);
      }
    }
  };
  auto store_a = [&](int buf, const uint4 (&v)[8]) {
    uint4* dst = (uint4*)(As + buf * BM * LDA + tid * LDA);
#pragma unroll
    for (int q = 0; q < 8; ++q) dst[q] = v[q];
  };
  const int b_row = n0 + tid;

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  {
    uint4 av[8];
    BStage<BITS> bs;
    load_a(0, av);
    load_b<BITS, ZK>(p, b_row, 0, bs);
    store_a(0, av);
    store_b<BITS>(bs, Bs + tid * LDA);
  }
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nsteps;
    uint4 av[8];
    BStage<BITS> bs;
    if (more) {
      load_a((s + 1) * BK, av);
      load_b<BITS, ZK>(p, b_row, (s + 1) * BK, bs);
    }
    const uint16_t* Ab = As + buf * BM * LDA;
    const uint16_t* Bb = Bs + buf * BN * LDA;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      f16x8 af[4], bf[4];
      const int koff = kk + 8 * (lane >> 5);
#pragma unroll
      for (int a = 0; a < 4; ++a)
        af[a] = *(const f16x8*)(Ab + (wm * 128 + a * 32 + (lane & 31)) * LDA + koff);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        bf[b] = *(const f16x8*)(Bb + (wn * 128 + b * 32 + (lane & 31)) * LDA + koff);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    if (more) {
      store_a(buf ^ 1, av);
      store_b<BITS>(bs, Bs + (buf ^ 1) * BN * LDA + tid * LDA);
    }
    __syncthreads();
  }

  // epilogue: + bias, convert, store (rows/columns past the end are skipped)
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int col = n0 + wn * 128 + b * 32 + (lane & 31);
    const bool col_ok = col < p.N;
    const float bv = (p.bias && col_ok) ? load_bias<CT>(p.bias, col) : 0.0f;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 128 + a * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (col_ok && row < p.M) store_c<CT>(p.C, (int64_t)row * p.N + col, acc[a][b][v] + bv);
      }
    }
  }
}

constexpr size_t kPrefillLds = (size_t)2 * (BM + BN) * LDA * sizeof(uint16_t);

template <int BITS, int ZK, int CT>
void launch_one(const PrefillArgs& p, dim3 grid, hipStream_t st) {
  auto k = prefill_kernel<BITS, ZK, CT>;
  static bool attr = false;  // per instantiation
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kPrefillLds);
    attr = true;
  }
  hipLaunchKernelGGL(k, grid, dim3(NT), kPrefillLds, st, p);
}

template <int BITS, int ZK>
void launch_ct(const PrefillArgs& p, dim3 grid, hipStream_t st) {
  if (p.c_type == QMM_F32) launch_one<BITS, ZK, QMM_F32>(p, grid, st);
  else if (p.c_type == QMM_F16) launch_one<BITS, ZK, QMM_F16>(p, grid, st);
  else launch_one<BITS, ZK, QMM_BF16>(p, grid, st);
}

}  // namespace

hipError_t launch_prefill(PrefillArgs p, hipStream_t st) {
  p.ntiles = (int)((p.N + BN - 1) / BN);
  p.mtiles = (int)((p.M + BM - 1) / BM);
  const int64_t groups = (p.ntiles + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * p.mtiles));
  const int zk = p.zp_kind == QMM_ZP_PACKED ? 1 : p.zp_kind == QMM_ZP_F16 ? 2 : 0;
  if (p.bits == 2) {
    if (zk == 1) launch_ct<2, 1>(p, grid, st);
    else if (zk == 2) launch_ct<2, 2>(p, grid, st);
    else launch_ct<2, 0>(p, grid, st);
  } else {
    if (zk == 1) launch_ct<4, 1>(p, grid, st);
    else if (zk == 2) launch_ct<4, 2>(p, grid, st);
    else launch_ct<4, 0>(p, grid, st);
  }
  return hipSuccess;
}

}  // namespace qmm
