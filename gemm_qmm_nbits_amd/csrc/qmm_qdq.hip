// Activation quantize / dequantize ops and the fused quantized SwiGLU
// ([P1] hip-ep PR 1318, "Why": the per-layer chain Q(gate) -> qsigmoid -> 2x qmul ->
// Q(up) -> DQ costs about ten launches and an integer tensor per step; "What",
// commit 4: a fused Q -> DQ round trip and a fused quantized SwiGLU, each exactly
// equal to the unfused chain).
//
// Every op works element by element with per-tensor (scale, zero point) and uint8
// (bits = 8) or uint16 (bits = 16) codes:
//   Q(x)     = min(max(rint(fp32(x / s)) + zp, 0), 2^bits - 1), a NaN quotient -> 0
//   DQ(q)    = fp32((q - zp) * s)
//   sigmoid  = fp32 of 1 / (1 + e^-v) evaluated in fp64
//   qmul     = Q(fp32(DQ(a) * DQ(b)))
// with correctly rounded fp32 divides and no contraction of the separate roundings.
// The unfused ops and the fused ones share these device functions, so the fused
// kernels give the bits of the chain by construction; the tests compare both against
// the oracle's chain.  The ops are HBM-bound: one pass over the inputs and outputs,
// each thread four consecutive elements (16-byte loads when every pointer allows).
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int kQdqThreads = 256;

__device__ __forceinline__ float q_code(float x, float s, float z, float qmax) {
  const float t = __fdiv_rn(x, s);
  const float r = __fadd_rn(rintf(t), z);  // exact below 2^24; saturates beyond
  return fminf(fmaxf(r, 0.0f), qmax);      // fmaxf(NaN, 0) = 0
}

__device__ __forceinline__ float dq_value(float q, float s, float z) { return __fmul_rn(__fsub_rn(q, z), s); }

__device__ __forceinline__ float sigmoid_f32(float v) {
  const double e = exp(-(double)v);
  return (float)(1.0 / (1.0 + e));
}

template <int T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  if constexpr (T == QMM_F32) return ((const float*)p)[i];
  else if constexpr (T == QMM_F16) return f16_to_f32(((const uint16_t*)p)[i]);
  else return bf16_to_f32(((const uint16_t*)p)[i]);
}

// A 16-bit output is the nearest value of the fp32 result: the empty asm makes the fp32
// value a register the conversion reads, so the compiler cannot merge the multiply
// that produced it and the conversion into one mixed-precision operation (which would
// round the exact product once to 16 bits and differ where the fp32 value falls on a
// 16-bit midpoint).
template <int T>
__device__ __forceinline__ void st(void* p, int64_t i, float v) {
  if constexpr (T == QMM_F32) {
    ((float*)p)[i] = v;
  } else {
    asm volatile("" : "+v"(v));
    if constexpr (T == QMM_F16) ((uint16_t*)p)[i] = f32_to_f16(v);
    else ((uint16_t*)p)[i] = f32_to_bf16(v);
  }
}

template <int BITS>
__device__ __forceinline__ float ldq(const void* p, int64_t i) {
  if constexpr (BITS == 8) return (float)((const uint8_t*)p)[i];
  else return (float)((const uint16_t*)p)[i];
}

template <int BITS>
__device__ __forceinline__ void stq(void* p, int64_t i, float q) {
  if constexpr (BITS == 8) ((uint8_t*)p)[i] = (uint8_t)q;
  else ((uint16_t*)p)[i] = (uint16_t)q;
}

// Four consecutive elements per thread; the element index of a thread's group is a
// multiple of 4, so per-element loads of a group are contiguous.
template <typename F>
__device__ __forceinline__ void for_each4(int64_t n, F&& f) {
  const int64_t groups = (n + 3) / 4;
  for (int64_t g = (int64_t)blockIdx.x * kQdqThreads + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * kQdqThreads) {
    const int64_t i0 = 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i0 + e < n) f(i0 + e);
  }
}

struct QP {
  float s, z, qmax;
};

template <int XT, int BITS>
__global__ __launch_bounds__(kQdqThreads) void quantize_kernel(const void* x, int64_t n, QP q, void* codes) {
  for_each4(n, [&](int64_t i) { stq<BITS>(codes, i, q_code(ld<XT>(x, i), q.s, q.z, q.qmax)); });
}

template <int BITS, int YT>
__global__ __launch_bounds__(kQdqThreads) void dequantize_kernel(const void* codes, int64_t n, QP q, void* y) {
  for_each4(n, [&](int64_t i) { st<YT>(y, i, dq_value(ldq<BITS>(codes, i), q.s, q.z)); });
}

template <int XT>
__global__ __launch_bounds__(kQdqThreads) void fake_quantize_kernel(const void* x, int64_t n, QP q, void* y) {
  for_each4(n, [&](int64_t i) { st<XT>(y, i, dq_value(q_code(ld<XT>(x, i), q.s, q.z, q.qmax), q.s, q.z)); });
}

template <int BITS>
__global__ __launch_bounds__(kQdqThreads) void qsigmoid_kernel(const void* in, int64_t n, QP qi, QP qo, void* out) {
  for_each4(n, [&](int64_t i) {
    const float v = dq_value(ldq<BITS>(in, i), qi.s, qi.z);
    stq<BITS>(out, i, q_code(sigmoid_f32(v), qo.s, qo.z, qo.qmax));
  });
}

template <int BITS>
__global__ __launch_bounds__(kQdqThreads) void qmul_kernel(const void* a, QP qa, const void* b, QP qb, int64_t n,
                                                           QP qc, void* c) {
  for_each4(n, [&](int64_t i) {
    const float p = __fmul_rn(dq_value(ldq<BITS>(a, i), qa.s, qa.z), dq_value(ldq<BITS>(b, i), qb.s, qb.z));
    stq<BITS>(c, i, q_code(p, qc.s, qc.z, qc.qmax));
  });
}

// The whole chain per element, in registers: gate and up are read once, y written once.
template <int XT, int BITS>
__global__ __launch_bounds__(kQdqThreads) void qswiglu_kernel(const void* gate, const void* up, int64_t n, QP qg,
                                                              QP qs, QP qm, QP qu, QP qh, void* y) {
  for_each4(n, [&](int64_t i) {
    const float g = q_code(ld<XT>(gate, i), qg.s, qg.z, qg.qmax);
    const float gd = dq_value(g, qg.s, qg.z);
    const float t = q_code(sigmoid_f32(gd), qs.s, qs.z, qs.qmax);
    const float m = q_code(__fmul_rn(gd, dq_value(t, qs.s, qs.z)), qm.s, qm.z, qm.qmax);
    const float u = q_code(ld<XT>(up, i), qu.s, qu.z, qu.qmax);
    const float h = q_code(__fmul_rn(dq_value(m, qm.s, qm.z), dq_value(u, qu.s, qu.z)), qh.s, qh.z, qh.qmax);
    st<XT>(y, i, dq_value(h, qh.s, qh.z));
  });
}

dim3 qdq_grid(int64_t n) {
  int64_t g = ((n + 3) / 4 + kQdqThreads - 1) / kQdqThreads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return dim3((unsigned)g);
}

QP qp_of(const QdqParams& p, int bits) { return QP{p.scale, (float)p.zero_point, (float)((1 << bits) - 1)}; }

template <int XT>
void q_at(const void* x, int64_t n, QP q, int bits, void* codes, hipStream_t st_) {
  if (bits == 8) launch((quantize_kernel<XT, 8>), qdq_grid(n), dim3(kQdqThreads), 0, st_, x, n, q, codes);
  else launch((quantize_kernel<XT, 16>), qdq_grid(n), dim3(kQdqThreads), 0, st_, x, n, q, codes);
}

template <int YT>
void dq_at(const void* codes, int64_t n, QP q, int bits, void* y, hipStream_t st_) {
  if (bits == 8) launch((dequantize_kernel<8, YT>), qdq_grid(n), dim3(kQdqThreads), 0, st_, codes, n, q, y);
  else launch((dequantize_kernel<16, YT>), qdq_grid(n), dim3(kQdqThreads), 0, st_, codes, n, q, y);
}

template <int XT>
void swiglu_at(const void* gate, const void* up, int64_t n, int bits, const QdqParams* p, void* y, hipStream_t st_) {
  const QP a = qp_of(p[0], bits), b = qp_of(p[1], bits), c = qp_of(p[2], bits), d = qp_of(p[3], bits),
           e = qp_of(p[4], bits);
  if (bits == 8)
    launch((qswiglu_kernel<XT, 8>), qdq_grid(n), dim3(kQdqThreads), 0, st_, gate, up, n, a, b, c, d, e, y);
  else
    launch((qswiglu_kernel<XT, 16>), qdq_grid(n), dim3(kQdqThreads), 0, st_, gate, up, n, a, b, c, d, e, y);
}

}  // namespace

hipError_t launch_quantize_linear(const void* x, int x_type, int64_t n, QdqParams q, int bits, void* codes,
                                  hipStream_t st_) {
  const QP p = qp_of(q, bits);
  if (x_type == QMM_F32) q_at<QMM_F32>(x, n, p, bits, codes, st_);
  else if (x_type == QMM_F16) q_at<QMM_F16>(x, n, p, bits, codes, st_);
  else q_at<QMM_BF16>(x, n, p, bits, codes, st_);
  return hipSuccess;
}

hipError_t launch_dequantize_linear(const void* codes, int64_t n, QdqParams q, int bits, void* y, int y_type,
                                    hipStream_t st_) {
  const QP p = qp_of(q, bits);
  if (y_type == QMM_F32) dq_at<QMM_F32>(codes, n, p, bits, y, st_);
  else if (y_type == QMM_F16) dq_at<QMM_F16>(codes, n, p, bits, y, st_);
  else dq_at<QMM_BF16>(codes, n, p, bits, y, st_);
  return hipSuccess;
}

hipError_t launch_fake_quantize(const void* x, int x_type, int64_t n, QdqParams q, int bits, void* y,
                                hipStream_t st_) {
  const QP p = qp_of(q, bits);
  if (x_type == QMM_F32)
    launch((fake_quantize_kernel<QMM_F32>), qdq_grid(n), dim3(kQdqThreads), 0, st_, x, n, p, y);
  else if (x_type == QMM_F16)
    launch((fake_quantize_kernel<QMM_F16>), qdq_grid(n), dim3(kQdqThreads), 0, st_, x, n, p, y);
  else
    launch((fake_quantize_kernel<QMM_BF16>), qdq_grid(n), dim3(kQdqThreads), 0, st_, x, n, p, y);
  return hipSuccess;
}

hipError_t launch_qsigmoid(const void* in, int64_t n, QdqParams qi, QdqParams qo, int bits, void* out,
                           hipStream_t st_) {
  const QP a = qp_of(qi, bits), b = qp_of(qo, bits);
  if (bits == 8) launch((qsigmoid_kernel<8>), qdq_grid(n), dim3(kQdqThreads), 0, st_, in, n, a, b, out);
  else launch((qsigmoid_kernel<16>), qdq_grid(n), dim3(kQdqThreads), 0, st_, in, n, a, b, out);
  return hipSuccess;
}

hipError_t launch_qmul(const void* a, QdqParams qa, const void* b, QdqParams qb, int64_t n, QdqParams qc, int bits,
                       void* c, hipStream_t st_) {
  const QP pa = qp_of(qa, bits), pb = qp_of(qb, bits), pc = qp_of(qc, bits);
  if (bits == 8)
    launch((qmul_kernel<8>), qdq_grid(n), dim3(kQdqThreads), 0, st_, a, pa, b, pb, n, pc, c);
  else
    launch((qmul_kernel<16>), qdq_grid(n), dim3(kQdqThreads), 0, st_, a, pa, b, pb, n, pc, c);
  return hipSuccess;
}

hipError_t launch_qswiglu(const void* gate, const void* up, int x_type, int64_t n, int bits, const QdqParams* q,
                          void* y, hipStream_t st_) {
  if (x_type == QMM_F32) swiglu_at<QMM_F32>(gate, up, n, bits, q, y, st_);
  else if (x_type == QMM_F16) swiglu_at<QMM_F16>(gate, up, n, bits, q, y, st_);
  else swiglu_at<QMM_BF16>(gate, up, n, bits, q, y, st_);
  return hipSuccess;
}

}  // namespace qmm
