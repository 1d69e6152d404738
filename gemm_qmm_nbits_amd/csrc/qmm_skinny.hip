// Skinny matrix-core path of MatMulNBits and the 16-entry codebook for 8 < M <= 64
// (activations of a few tokens: [P1] hip-ep PR 1318 "What", the prefill tiles on the
// matrix cores with A cast to fp16 once; [P3] bitsandbytes PR 1979 "Technical
// details", the codebook decoded inside the matrix product).
//
// C[M][N] = A16 . W16^T (+ bias) with the operand roundings of the prefill path:
// A16 = fp16(A) (cast once into the caller's workspace, rows zero-padded to Kp, a
// multiple of 64) and W16 = fp16 of the exact fp32 dequantized weight
// (fp32(fp32(q - zp) * s) or fp32(codebook[q] * absmax)).  Unlike the 256 x 256 prefill
// tiles, no matrix-core work is spent on padding rows beyond ceil(M / 16) * 16, and every
// weight is loaded and dequantized once.
//
// Work-group: 8 waves and one, two or four 16-row strips of W (16 to 64 output columns).  The reduction
// runs in steps of 128 codes; wave w takes steps w, w + 8, ...  In a step, lane l
// (n = l % 16, q = l / 16) loads codes [32q, 32q + 32) of W row n of each strip (8 bytes
// of u2, 12 of u3, 16 of u4, 32 of i8, inside one block since blocks are >= 32 codes),
// dequantizes them into
// four groups of 8 fp16, and reads the matching 8 fp16 of A for each 16-row M tile
// straight from the workspace (L2-resident).  v_mfma_f32_16x16x32_f16 then contracts the
// 8-value groups: lane l supplies A row l % 16 and W row l % 16 over the same 8 k, so
// the pairing is exact whatever order the instruction takes its k in; accumulator v of
// lane l is row 4 * (l / 16) + v, column l % 16.  The eight waves' fp32 sums are added
// in wave order through LDS.  When the grid would not fill the chip, the reduction is
// split into contiguous step ranges whose fp32 partial sums the split reduction adds in
// order.  The result depends only on the shape.
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_skinny.h"

namespace qmm {

namespace {

constexpr int SK_WAVES = 8;
constexpr int SK_THREADS = SK_WAVES * 64;
// NS: 16-row strips of W per work-group.  More strips let each activation fragment
// feed more matrix-core steps; fewer give a narrow output more work-groups.  One M
// tile: one strip when N / 16 work-groups fit on the compute units in one round, else
// two.  Two or four M tiles: four strips when N / 64 work-groups still cover three
// quarters of the compute units, else two.  (Measured on MI355X at the 16-entry
// codebook shapes, M = 16 and 64.)  The strip count never changes any output's
// summation order.
constexpr int SK_STEP = 128;   // codes per reduction step
constexpr uint32_t kSkWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const void* p, int64_t bytes) {
  const uint32_t n = bytes >= 0x7fffffff ? 0x7fffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, (int)kSkWord3);
}

template <int CT>
__device__ __forceinline__ void sk_store(void* C, int64_t i, float v) {
  if constexpr (CT == QMM_F32) ((float*)C)[i] = v;
  else if constexpr (CT == QMM_F16) ((uint16_t*)C)[i] = f32_to_f16(v);
  else ((uint16_t*)C)[i] = f32_to_bf16(v);
}

template <int CT>
__device__ __forceinline__ float sk_bias(const void* b, int64_t i) {
  if constexpr (CT == QMM_F32) return ((const float*)b)[i];
  else if constexpr (CT == QMM_F16) return f16_to_f32(((const uint16_t*)b)[i]);
  else return bf16_to_f32(((const uint16_t*)b)[i]);
}

// 8 codes -> 8 fp16 weights (codes in order), exact fp32 dequant rounded to nearest
// fp16.  BITS = 4: `xw` holds the 8 codes as nibbles; BITS = 2: in its low 16 bits;
// BITS = 3: in its low 24 bits; BITS = 8: four signed bytes in xw, four in xw2.
// fz: q - z is exact for every code and z * sc is exact (integer zero points, or a
// constant that passed zconst_fma_exact), so fp32((q - z) * sc) is one fma.
template <int FMT, int BITS>
__device__ __forceinline__ f16x8 dequant8(uint32_t xw, uint32_t xw2, float sc, float z, float am,
                                          const float* cb, bool fz) {
  uint32_t o[4];
  if constexpr (FMT == GEMV_CODEBOOK) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x2 w;
      w.x = __fmul_rn(cb[(xw >> (8 * jj)) & 15u], am);
      w.y = __fmul_rn(cb[(xw >> (8 * jj + 4)) & 15u], am);
      o[jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2));
    }
  } else {
    // codes as exact fp32 integers, two per conversion: 2-bit codes masked into e2m1
    // nibbles are q/2 (scaled by 2), 4-bit codes masked into e4m3 bytes are q * 2^-9
    // (scaled by 2^9)
    float qv[8];
    if constexpr (BITS == 3) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = (float)__builtin_amdgcn_ubfe(xw, 3 * i, 3);
    } else if constexpr (BITS == 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[i] = (float)(int)__builtin_amdgcn_sbfe((int)xw, 8 * i, 8);
        qv[4 + i] = (float)(int)__builtin_amdgcn_sbfe((int)xw2, 8 * i, 8);
      }
    } else if constexpr (BITS == 2) {
      const uint32_t ev = xw & 0x3333u, od = (xw >> 2) & 0x3333u;
      const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 2.0f, 0);
      const f32x2 o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 2.0f, 0);
      const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 2.0f, 1);
      const f32x2 o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 2.0f, 1);
      qv[0] = e0.x; qv[2] = e0.y; qv[1] = o0.x; qv[3] = o0.y;
      qv[4] = e1.x; qv[6] = e1.y; qv[5] = o1.x; qv[7] = o1.y;
    } else {
      const uint32_t lo = xw & 0x0F0F0F0Fu, hi = (xw >> 4) & 0x0F0F0F0Fu;
      const f32x2 l0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, false);
      const f32x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, false);
      const f32x2 l1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, true);
      const f32x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, true);
      qv[0] = l0.x; qv[2] = l0.y; qv[4] = l1.x; qv[6] = l1.y;
      qv[1] = h0.x; qv[3] = h0.y; qv[5] = h1.x; qv[7] = h1.y;
    }
    if (fz) {
      const float nzs = -(z * sc);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x2 w;
        w.x = __fmaf_rn(qv[2 * jj], sc, nzs);
        w.y = __fmaf_rn(qv[2 * jj + 1], sc, nzs);
        o[jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2));  // nearest even
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x2 w;
        w.x = __fmul_rn(__fsub_rn(qv[2 * jj], z), sc);
        w.y = __fmul_rn(__fsub_rn(qv[2 * jj + 1], z), sc);
        o[jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2));  // nearest even
      }
    }
  }
  return __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// FMT: GEMV_AFFINE (w = (q - zp) * s) or GEMV_CODEBOOK (BITS = 4); MB: 16-row M tiles.
template <int FMT, int BITS, int ZK, int CT, int MB, int SK_NS>
__global__ __launch_bounds__(SK_THREADS) void skinny_kernel(PrefillArgs p) {
  __shared__ float cb[16];
  extern __shared__ float red[];  // [SK_WAVES][MB * SK_NS * 4][64]
  if constexpr (FMT == GEMV_CODEBOOK) {
    if (threadIdx.x < 16) cb[threadIdx.x] = p.codebook[threadIdx.x];
    __syncthreads();
  }
  const int wave = (int)(threadIdx.x >> 6);
  const int lane = (int)(threadIdx.x & 63);
  const int ln = lane & 15, lq = lane >> 4;
  const int M = (int)p.M, N = (int)p.N, Kp = (int)p.Kp;
  const int nsteps = (Kp + SK_STEP - 1) / SK_STEP;
  const int nblk = (int)p.nblk, blog = p.block_log2;
  const int n0 = (int)blockIdx.x * (SK_NS * 16);
  // reduction split ks covers steps [ks * spl, (ks + 1) * spl)
  const int ks = (int)blockIdx.y;
  const int s_begin = ks * p.spl;
  const int s_end = s_begin + p.spl < nsteps ? s_begin + p.spl : nsteps;

  const __amdgpu_buffer_rsrc_t rW = sk_rsrc(p.W, p.N * p.row_bytes);
  const __amdgpu_buffer_rsrc_t rS = FMT == GEMV_CODEBOOK ? sk_rsrc(p.absmax, p.N * p.nblk * 4)
                                                          : sk_rsrc(p.scales, p.N * p.nblk * 2);
  __amdgpu_buffer_rsrc_t rZ = rS;
  if constexpr (ZK == 1) rZ = sk_rsrc(p.zp, p.N * p.zp_row_bytes);
  if constexpr (ZK == 2) rZ = sk_rsrc(p.zp, p.N * p.nblk * 2);
  // A rows past M lie past the buffer's range and read as zero
  const __amdgpu_buffer_rsrc_t rA = sk_rsrc(p.A16, (int64_t)p.M * p.lda * 2);
  const int lda = (int)p.lda;
  // activations at k >= K8 (K rounded up to 8) read as zero: the cast workspace holds
  // zeros there anyway; fp16 A read in place (K % 8 == 0) would hold the next row
  const int K8 = (int)((p.K + 7) / 8 * 8);

  // W rows of this lane (clamped: rows past N are computed and dropped)
  uint32_t wrow[SK_NS];
#pragma unroll
  for (int s = 0; s < SK_NS; ++s) {
    const int n = n0 + s * 16 + ln;
    wrow[s] = (uint32_t)(n < N ? n : N - 1);
  }

  f32x4 acc[MB][SK_NS];
#pragma unroll
  for (int mt = 0; mt < MB; ++mt)
#pragma unroll
    for (int s = 0; s < SK_NS; ++s) acc[mt][s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int c = s_begin + wave; c < s_end; c += SK_WAVES) {
    const int k0 = c * SK_STEP + lq * 32;  // this lane's 32 codes
    const bool kin = k0 < Kp;             // Kp % 64 == 0: wholly inside or wholly past
    // weights: 32 codes, scale (or absmax) and zero point of their block, per strip
    uint32_t wv[SK_NS][BITS];
    float sc[SK_NS], z[SK_NS], am[SK_NS];
    int blk = k0 >> blog;
    blk = blk < nblk - 1 ? blk : nblk - 1;  // codes past the row end meet zero A
#pragma unroll
    for (int s = 0; s < SK_NS; ++s) {
      const uint32_t wo = wrow[s] * (uint32_t)p.row_bytes + (uint32_t)(k0 * BITS / 8);
      if constexpr (BITS == 8) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)wo, 0, 0);
        const auto u = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)(wo + 16u), 0, 0);
        wv[s][0] = v[0]; wv[s][1] = v[1]; wv[s][2] = v[2]; wv[s][3] = v[3];
        wv[s][4] = u[0]; wv[s][5] = u[1]; wv[s][6] = u[2]; wv[s][7] = u[3];
      } else if constexpr (BITS == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)wo, 0, 0);
        wv[s][0] = v[0]; wv[s][1] = v[1]; wv[s][2] = v[2]; wv[s][3] = v[3];
      } else if constexpr (BITS == 3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(rW, (int)wo, 0, 0);
        wv[s][0] = v[0]; wv[s][1] = v[1]; wv[s][2] = v[2];
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rW, (int)wo, 0, 0);
        wv[s][0] = v[0]; wv[s][1] = v[1];
      }
      const uint32_t sb = wrow[s] * (uint32_t)nblk + (uint32_t)blk;
      sc[s] = 0.0f; z[s] = 0.0f; am[s] = 0.0f;
      if constexpr (FMT == GEMV_CODEBOOK) {
        am[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, (int)(4u * sb), 0, 0));
      } else {
        sc[s] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rS, (int)(2u * sb), 0, 0));
        if constexpr (ZK == 1) {
          const int bit = blk * BITS;
          const uint32_t zo = wrow[s] * (uint32_t)p.zp_row_bytes + (uint32_t)(bit >> 3);
          uint32_t zb = __builtin_amdgcn_raw_buffer_load_b8(rZ, (int)zo, 0, 0);
          if constexpr (BITS == 8) {
            z[s] = (float)(int8_t)zb;
          } else {
            // a 3-bit field may continue into the next byte (past the buffer it reads 0)
            if constexpr (BITS == 3) zb |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rZ, (int)(zo + 1u), 0, 0) << 8;
            z[s] = (float)((zb >> (bit & 7)) & ((1u << BITS) - 1u));
          }
        } else if constexpr (ZK == 2) {
          z[s] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rZ, (int)(2u * sb), 0, 0));
        } else {
          z[s] = p.zconst;
        }
      }
    }
    // activations: 32 fp16 of row 16 mt + ln per M tile (zero past K8 and past M)
    f16x8 af[MB][4];
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) {
      const uint32_t ao = ((uint32_t)(mt * 16 + ln) * (uint32_t)lda + (uint32_t)(kin ? k0 : 0)) * 2u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool kj = kin && k0 + 8 * j < K8;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rA, (int)(kj ? ao + 16u * j : 0u), 0, 0);
        const uint4 u = kj ? make_uint4(v[0], v[1], v[2], v[3]) : make_uint4(0u, 0u, 0u, 0u);
        af[mt][j] = __builtin_bit_cast(f16x8, u);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int s = 0; s < SK_NS; ++s) {
        uint32_t xw, xw2 = 0u;
        if constexpr (BITS == 4) xw = wv[s][j];
        else if constexpr (BITS == 2) xw = wv[s][j >> 1] >> (16 * (j & 1));
        else if constexpr (BITS == 8) xw = wv[s][2 * j], xw2 = wv[s][2 * j + 1];
        else  // 3 bits: the 24-bit field at bit 24 j of the 96-bit group
          xw = j == 0 ? wv[s][0] : j == 1 ? __builtin_amdgcn_alignbit(wv[s][1], wv[s][0], 24)
             : j == 2 ? __builtin_amdgcn_alignbit(wv[s][2], wv[s][1], 16) : (wv[s][2] >> 8);
        const f16x8 bf = dequant8<FMT, BITS>(xw, xw2, sc[s], z[s], am[s], cb, ZK == 1 || (ZK == 0 && p.zconst_fma));
#pragma unroll
        for (int mt = 0; mt < MB; ++mt)
          acc[mt][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt][j], bf, acc[mt][s], 0, 0, 0);
      }
    }
  }

  // the eight waves' sums, added in wave order
  constexpr int R = MB * SK_NS * 4;
#pragma unroll
  for (int mt = 0; mt < MB; ++mt)
#pragma unroll
    for (int s = 0; s < SK_NS; ++s)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[((wave * R) + (mt * SK_NS + s) * 4 + v) * 64 + lane] = acc[mt][s][v];
  __syncthreads();
  for (int e = (int)threadIdx.x; e < R * 64; e += SK_THREADS) {
    const int r = e >> 6, l = e & 63;
    const int mt = r / (SK_NS * 4), s = (r >> 2) % SK_NS, v = r & 3;
    const int m = mt * 16 + 4 * (l >> 4) + v;
    const int n = n0 + s * 16 + (l & 15);
    if (m >= M || n >= N) continue;
    float y = red[r * 64 + l];
#pragma unroll
    for (int w = 1; w < SK_WAVES; ++w) y += red[(w * R + r) * 64 + l];
    if (p.splits > 1) {
      // fp32 partial sum of this split; the split reduction adds the splits in order
      p.partials[((int64_t)ks * M + m) * p.ldc + n] = y;
      continue;
    }
    if (p.row_scale) y *= p.row_scale[m];
    if (p.bias) y += sk_bias<CT>(p.bias, n);
    sk_store<CT>(p.C, (int64_t)m * p.ldc + n, y);
  }
}

template <int FMT, int BITS, int ZK, int CT, int MB, int SK_NS>
void sk_launch(const PrefillArgs& p, hipStream_t st) {
  auto kern = skinny_kernel<FMT, BITS, ZK, CT, MB, SK_NS>;
  const size_t lds = (size_t)SK_WAVES * MB * SK_NS * 4 * 64 * sizeof(float);
  if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const unsigned grid = (unsigned)((p.N + SK_NS * 16 - 1) / (SK_NS * 16));
  launch(kern, dim3(grid, (unsigned)p.splits), dim3(SK_THREADS), lds, st, p);
}

template <int FMT, int BITS, int ZK, int CT>
void sk_mb(const PrefillArgs& p, hipStream_t st) {
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
    (void)hipGetLastError();
    cus = 256;
  }
  if (p.M <= 16) {
    // one strip while the work-groups fit in one round; else four strips when that
    // still leaves three quarters of the compute units a work-group (one round, where
    // two strips would take nearly two), else two
    if ((p.N + 15) / 16 <= cus) sk_launch<FMT, BITS, ZK, CT, 1, 1>(p, st);
    else if ((p.N + 63) / 64 * 4 >= 3 * (int64_t)cus) sk_launch<FMT, BITS, ZK, CT, 1, 4>(p, st);
    else sk_launch<FMT, BITS, ZK, CT, 1, 2>(p, st);
  } else {
    // four strips (half the activation reads per matrix-core step) while that still
    // leaves at least three quarters of the compute units a work-group; one strip for
    // narrow outputs (N / 16 work-groups within half the compute units), whose split
    // reduction then fills the device, and for reductions too short to split when N / 16
    // work-groups fit on the compute units; else two
    const bool wide = (p.N + 63) / 64 * 4 >= 3 * (int64_t)cus;
    const int64_t nsteps = (p.Kp + SK_STEP - 1) / SK_STEP;
    const bool narrow = (p.N + 15) / 16 * 2 <= (int64_t)cus ||
                        (nsteps < 2 * SK_WAVES && (p.N + 15) / 16 <= (int64_t)cus);
    if (p.M <= 32) {
      if (wide) sk_launch<FMT, BITS, ZK, CT, 2, 4>(p, st);
      else if (narrow) sk_launch<FMT, BITS, ZK, CT, 2, 1>(p, st);
      else sk_launch<FMT, BITS, ZK, CT, 2, 2>(p, st);
    } else {
      if (wide) sk_launch<FMT, BITS, ZK, CT, 4, 4>(p, st);
      else if (narrow) sk_launch<FMT, BITS, ZK, CT, 4, 1>(p, st);
      else sk_launch<FMT, BITS, ZK, CT, 4, 2>(p, st);
    }
  }
}

template <int FMT, int BITS, int ZK>
void sk_ct(const PrefillArgs& p, hipStream_t st) {
  if (p.c_type == QMM_F32) sk_mb<FMT, BITS, ZK, QMM_F32>(p, st);
  else if (p.c_type == QMM_F16) sk_mb<FMT, BITS, ZK, QMM_F16>(p, st);
  else sk_mb<FMT, BITS, ZK, QMM_BF16>(p, st);
}


// ---- ragged multi-token MoE matmul -------------------------------------------------
//
// Rows of X are grouped by expert (expert e owns rows offsets[e] .. offsets[e+1]-1), and
// Y[r] = fp16(X[r] . W16_e^T + b_e) with the operands of the skinny kernel: fp16 X as
// given and W16 = fp16 of the exact fp32 dequant.  Work-group slot y is the y-th tile of
// 16 * MB rows in expert order (each expert's rows split into tiles, empty experts none);
// wave 0 finds the slot's expert by a prefix sum of the experts' tile counts, and slots
// past the last tile exit.  Within a tile the work is the skinny kernel's: 8 waves take
// 128-code steps, lane l loads 32 codes of W_e row n0 + 16 s + l % 16 per strip s and 8
// fp16 of X row l % 16 of each 16-row M tile (rows of the next expert and k >= K read
// as zero), v_mfma_f32_16x16x32_f16 accumulates, and the waves' sums are added in wave
// order.  The summation order depends only on K.
template <int ZK, int MB, int NS>
__global__ __launch_bounds__(SK_THREADS) void ragged_kernel(RaggedArgs p) {
  extern __shared__ float red[];  // [SK_WAVES][MB * NS * 4][64]
  __shared__ int slot_expert, slot_tile;
  const int wave = (int)(threadIdx.x >> 6);
  const int lane = (int)(threadIdx.x & 63);
  const int ln = lane & 15, lq = lane >> 4;
  const int R = (int)p.R, E = (int)p.E, N = (int)p.N, K = (int)p.K;
  constexpr int kTileRows = 16 * MB;
  // offsets are clamped into [0, R] and made nondecreasing, so every row index stays in X
  auto off = [&](int e) {
    const int o = p.offsets[e];
    return o < 0 ? 0 : o > R ? R : o;
  };
  if (wave == 0) {
    const int slot = (int)blockIdx.y;
    int found_e = -1, found_t = 0, base = 0;
    for (int c = 0; c < E && found_e < 0; c += 64) {  // uniform over the wave
      const int e = c + lane;
      int tiles = 0;
      if (e < E) {
        const int o0 = off(e), o1 = off(e + 1);
        tiles = o1 > o0 ? (o1 - o0 + kTileRows - 1) / kTileRows : 0;
      }
      int incl = tiles;  // inclusive prefix over the lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        incl += lane >= d ? v : 0;
      }
      const int excl = incl - tiles;
      const bool mine = e < E && slot >= base + excl && slot < base + incl;
      const unsigned long long m = __ballot(mine);
      if (m) {
        const int src = __ffsll((long long)m) - 1;
        found_e = c + src;
        found_t = slot - base - __shfl(excl, src, 64);
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      slot_expert = found_e;
      slot_tile = found_t;
    }
  }
  __syncthreads();
  const int e = slot_expert;
  if (e < 0) return;  // past the last tile (uniform over the work-group)
  const int o0 = off(e), o1e = off(e + 1);
  const int o1 = o1e > o0 ? o1e : o0;
  const int r_begin = o0 + slot_tile * kTileRows;
  const int r_end = r_begin + kTileRows < o1 ? r_begin + kTileRows : o1;

  const int nblk = (int)p.nblk, blog = p.block_log2;
  const int nsteps = (K + SK_STEP - 1) / SK_STEP;
  const int n0 = (int)blockIdx.x * (NS * 16);
  const int64_t ew = (int64_t)e * p.N;  // first W row of expert e
  const __amdgpu_buffer_rsrc_t rW = sk_rsrc(p.W + ew * p.row_bytes, p.N * p.row_bytes);
  const __amdgpu_buffer_rsrc_t rS = sk_rsrc(p.scales + ew * nblk, p.N * p.nblk * 2);
  __amdgpu_buffer_rsrc_t rZ = rS;
  if constexpr (ZK == 1) rZ = sk_rsrc(p.zp + ew * p.zp_row_bytes, p.N * p.zp_row_bytes);
  const __amdgpu_buffer_rsrc_t rA = sk_rsrc(p.X, p.R * p.K * 2);

  uint32_t wrow[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int n = n0 + s * 16 + ln;
    wrow[s] = (uint32_t)(n < N ? n : N - 1);
  }
  // X rows of this lane per M tile, or -1 past the tile's rows
  int arow[MB];
#pragma unroll
  for (int mt = 0; mt < MB; ++mt) {
    const int r = r_begin + mt * 16 + ln;
    arow[mt] = r < r_end ? r : -1;
  }

  f32x4 acc[MB][NS];
#pragma unroll
  for (int mt = 0; mt < MB; ++mt)
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[mt][s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int c = wave; c < nsteps; c += SK_WAVES) {
    const int k0 = c * SK_STEP + lq * 32;  // this lane's 32 codes
    uint32_t wv[NS][4];
    float sc[NS], z[NS];
    int blk = k0 >> blog;
    blk = blk < nblk - 1 ? blk : nblk - 1;  // codes past the row end meet zero X
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t wo = wrow[s] * (uint32_t)p.row_bytes + (uint32_t)(k0 / 2);
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, (int)wo, 0, 0);
      wv[s][0] = v[0]; wv[s][1] = v[1]; wv[s][2] = v[2]; wv[s][3] = v[3];
      const uint32_t sb = wrow[s] * (uint32_t)nblk + (uint32_t)blk;
      sc[s] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rS, (int)(2u * sb), 0, 0));
      if constexpr (ZK == 1) {
        const uint32_t zb = __builtin_amdgcn_raw_buffer_load_b8(
            rZ, (int)(wrow[s] * (uint32_t)p.zp_row_bytes + (uint32_t)(blk >> 1)), 0, 0);
        z[s] = (float)((zb >> (4 * (blk & 1))) & 15u);
      } else {
        z[s] = 8.0f;
      }
    }
    f16x8 af[MB][4];
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = arow[mt] >= 0 && k0 + 8 * j < K;
        const uint32_t ao = ok ? ((uint32_t)arow[mt] * (uint32_t)K + (uint32_t)(k0 + 8 * j)) * 2u : 0u;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rA, (int)ao, 0, 0);
        const uint4 u = ok ? make_uint4(v[0], v[1], v[2], v[3]) : make_uint4(0u, 0u, 0u, 0u);
        af[mt][j] = __builtin_bit_cast(f16x8, u);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const f16x8 bf = dequant8<GEMV_AFFINE, 4>(wv[s][j], 0u, sc[s], z[s], 0.0f, nullptr, true);
#pragma unroll
        for (int mt = 0; mt < MB; ++mt)
          acc[mt][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt][j], bf, acc[mt][s], 0, 0, 0);
      }
    }
  }

  constexpr int RR = MB * NS * 4;
#pragma unroll
  for (int mt = 0; mt < MB; ++mt)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[((wave * RR) + (mt * NS + s) * 4 + v) * 64 + lane] = acc[mt][s][v];
  __syncthreads();
  const uint16_t* bias = p.bias ? p.bias + ew : nullptr;
  for (int i = (int)threadIdx.x; i < RR * 64; i += SK_THREADS) {
    const int r = i >> 6, l = i & 63;
    const int mt = r / (NS * 4), s = (r >> 2) % NS, v = r & 3;
    const int row = r_begin + mt * 16 + 4 * (l >> 4) + v;
    const int n = n0 + s * 16 + (l & 15);
    if (row >= r_end || n >= N) continue;
    float y = red[r * 64 + l];
#pragma unroll
    for (int w = 1; w < SK_WAVES; ++w) y += red[(w * RR + r) * 64 + l];
    if (bias) y += f16_to_f32(bias[n]);
    p.Y[(int64_t)row * N + n] = f32_to_f16(y);
  }
}

template <int ZK, int MB, int NS>
void ragged_launch(const RaggedArgs& p, hipStream_t st) {
  auto kern = ragged_kernel<ZK, MB, NS>;
  const size_t lds = (size_t)SK_WAVES * MB * NS * 4 * 64 * sizeof(float);
  if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const unsigned gx = (unsigned)((p.N + NS * 16 - 1) / (NS * 16));
  // every expert's tiles, at most ceil(R / rows) + E slots
  const unsigned gy = (unsigned)((p.R + 16 * MB - 1) / (16 * MB) + p.E);
  launch(kern, dim3(gx, gy), dim3(SK_THREADS), lds, st, p);
}

template <int ZK>
void ragged_mb(const RaggedArgs& p, hipStream_t st) {
  // tile height from the mean rows per expert: one 16-row tile for sparse bursts, up to
  // four when experts hold many rows (each weight strip then feeds more MFMA steps)
  const int64_t mean = p.E > 0 ? (p.R + p.E - 1) / p.E : p.R;
  const bool wide = p.N >= 2048;
  if (mean <= 16) wide ? ragged_launch<ZK, 1, 2>(p, st) : ragged_launch<ZK, 1, 1>(p, st);
  else if (mean <= 32) wide ? ragged_launch<ZK, 2, 2>(p, st) : ragged_launch<ZK, 2, 1>(p, st);
  else wide ? ragged_launch<ZK, 4, 2>(p, st) : ragged_launch<ZK, 4, 1>(p, st);
}

}  // namespace

hipError_t launch_ragged(const RaggedArgs& p, hipStream_t st) {
  if (p.zp) ragged_mb<1>(p, st);
  else ragged_mb<0>(p, st);
  return hipSuccess;
}

bool skinny_applies(int64_t M, int64_t N, int64_t Kp, int block, int64_t row_bytes, int64_t nblk) {
  // 32-bit buffer offsets for W, scales and the workspace rows
  if (M > kSkinnyMaxM || block < 32 || Kp <= 0) return false;
  // (activation offsets are formed for all 16 * ceil(M / 16) <= 64 tile rows)
  if (N * row_bytes >= (1LL << 31) || N * nblk * 4 >= (1LL << 31) || 64 * (Kp + 128) * 2 >= (1LL << 31))
    return false;
  return true;
}

int skinny_splits(int64_t M, int64_t N, int64_t Kp) {
  // Split the reduction while the grid stays within one work-group per compute unit
  // of a 256-CU device (work-groups counted as the launch deals strips on such a
  // device) and every wave of a split keeps at least one step; powers of two up to 8.
  // The partial sums go to the workspace, which holds prefill_splits(M, N, Kp) of them.
  const bool wide = (N + 63) / 64 * 4 >= 3 * 256;
  const int64_t nsteps = (Kp + SK_STEP - 1) / SK_STEP;
  const bool narrow = (N + 15) / 16 * 2 <= 256 || (nsteps < 2 * SK_WAVES && (N + 15) / 16 <= 256);
  const int64_t wgs = (M <= 16 && (N + 15) / 16 <= 256) ? (N + 15) / 16
                      : wide                             ? (N + 63) / 64
                      : narrow                           ? (N + 15) / 16
                                                         : (N + 31) / 32;
  const int64_t cap = prefill_splits(M, N, Kp);
  int s = 1;
  while (s < 8 && wgs * s * 2 <= 256 && nsteps >= (int64_t)s * 2 * SK_WAVES && s * 2 <= cap) s *= 2;
  return s;
}

hipError_t launch_skinny(const PrefillArgs& p0, hipStream_t st) {
  PrefillArgs p = p0;
  const int64_t nsteps = (p.Kp + SK_STEP - 1) / SK_STEP;
  p.splits = p.partials ? skinny_splits(p.M, p.N, p.Kp) : 1;
  p.spl = (int)((nsteps + p.splits - 1) / p.splits);
  const int zk = p.zp_kind == QMM_ZP_PACKED ? 1 : p.zp_kind == QMM_ZP_F16 ? 2 : 0;
  if (p.fmt == GEMV_CODEBOOK) {
    sk_ct<GEMV_CODEBOOK, 4, 0>(p, st);
  } else if (p.bits == 2) {
    if (zk == 1) sk_ct<GEMV_AFFINE, 2, 1>(p, st);
    else if (zk == 2) sk_ct<GEMV_AFFINE, 2, 2>(p, st);
    else sk_ct<GEMV_AFFINE, 2, 0>(p, st);
  } else if (p.bits == 3) {
    if (zk == 1) sk_ct<GEMV_AFFINE, 3, 1>(p, st);
    else if (zk == 2) sk_ct<GEMV_AFFINE, 3, 2>(p, st);
    else sk_ct<GEMV_AFFINE, 3, 0>(p, st);
  } else if (p.bits == 8) {
    if (zk == 1) sk_ct<GEMV_AFFINE, 8, 1>(p, st);
    else if (zk == 2) sk_ct<GEMV_AFFINE, 8, 2>(p, st);
    else sk_ct<GEMV_AFFINE, 8, 0>(p, st);
  } else {
    if (zk == 1) sk_ct<GEMV_AFFINE, 4, 1>(p, st);
    else if (zk == 2) sk_ct<GEMV_AFFINE, 4, 2>(p, st);
    else sk_ct<GEMV_AFFINE, 4, 0>(p, st);
  }
  if (p.splits > 1)
    return launch_reduce_splits(p.partials, p.splits, p.M, p.N, p.ldc, p.row_scale, p.bias, p.C, p.c_type, st);
  return hipSuccess;
}

}  // namespace qmm
