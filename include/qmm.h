/*
 * qmm.h -- C ABI of the fused low-bit dequantize-matmul library for MI355X (gfx950).
 *
 * The operations follow three public pages:
 *   [P1] hip-ep pull request 1318, "bits=2 MatMulNBits" (2-bit phi4-14B): sections
 *        "Why" and "What", commit 1 -- MatMulNBits with per-block fp16 scales and
 *        a zero point that is a tensor or, when all equal, a scalar; a GEMV that
 *        reads fp32 A and writes fp32 C; prefill tiles that cast A to fp16 once.
 *   [P2] hip-ep pull request 1328, "fused QMoE decode picks tiling up front":
 *        sections "Summary", "Why", "What", "Notes for reviewers" -- the top-k MoE
 *        decode fc1 -> SwiGLU -> fc2 with an int8-activation variant, tiling chosen
 *        before the first call computes, HIP error state cleared on entry,
 *        num_experts argument, scratch-only timing, capture fallback.
 *   [P3] bitsandbytes pull request 1979, "[ROCm] Fused 4-bit SIMT GEMM":
 *        sections "Summary" and "Technical details" -- 16-entry codebook (NF4/FP4)
 *        4-bit weights with per-block absmax, decoded inside the GEMM; A must be
 *        contiguous row-major.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps no reference to them after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Compute entry points only enqueue work on it and return without waiting,
 *     except the first call of a new shape, which times tiling candidates first
 *     (synchronizing the stream; never while the stream is being captured).
 *   - On entry the sticky HIP error state is cleared (hipGetLastError), so an
 *     error left by unrelated earlier work is not reported as this call's.
 *   - Return value (qmm_status): 0 on success; a negative QMM_E_* code if the
 *     arguments were refused before anything was launched; a positive value is
 *     the hipError_t reported after the launches.
 *   - Matrices are dense and row-major: A[M][K] (row stride K), C[M][N].
 *   - Packed weights: W[N][nblk][block*bits/8] bytes, nblk = ceil(K/block).
 *     Element k of row n lives in block b = k/block at position j = k%block, as
 *     the `bits`-wide field starting at bit j*bits of the block's little-endian
 *     bit stream (bit i of byte m is stream bit 8m + i; least significant field
 *     first, so a 3-bit field may continue into the next byte).  Codes of 2, 3 and
 *     4 bits are unsigned; 8-bit codes are signed bytes (two's complement). Codes
 *     past K in the last block are padding and are never read.
 *   - Dequantized weight (affine): w = fp32(fp32(q - zp) * fp32(scale)).
 *     Dequantized weight (codebook): w = fp32(codebook[q] * absmax).
 *   - Outputs are accumulated in fp32 and rounded once to the output dtype.
 *     Repeated calls with the same inputs give bit-identical outputs; the
 *     summation order depends only on (M-path, K, block, bits), never on the
 *     tiling chosen by the tuner.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int qmm_status;

/* element types */
enum { QMM_F32 = 0, QMM_F16 = 1, QMM_BF16 = 2 };

/* zero-point kinds ([P1] "What", commit 1) */
enum {
  QMM_ZP_NONE = 0,     /* zp = 2^(bits-1) for every block (0 for signed 8-bit codes)  */
  QMM_ZP_PACKED = 1,   /* uint8 [N][ceil(nblk*bits/8)]: codes in W's field layout (signed
                          bytes for 8-bit weights)                                      */
  QMM_ZP_F16 = 2,      /* fp16 [N][nblk]                                              */
  QMM_ZP_UNIFORM = 3   /* the scalar `uniform_zp`; the zp pointer is never read       */
};

/* MoE decode modes ([P2] "Summary": fp decode and its dp4a variant) */
enum { QMOE_FP = 0, QMOE_INT8_ACT = 1 };

/* refusal codes (negative): nothing was launched */
enum {
  QMM_OK = 0,
  QMM_E_NULL = -1,       /* a required pointer is NULL                                  */
  QMM_E_DTYPE = -2,      /* unsupported element type                                    */
  QMM_E_BITS = -3,       /* bits not in {2, 3, 4, 8} (MoE: 4; activation ops: 8, 16)    */
  QMM_E_BLOCK = -4,      /* block not a power of two in [16, 256] (3-bit weights and
                            MoE: >= 32)                                                 */
  QMM_E_SHAPE = -5,      /* a size is negative or out of range                          */
  QMM_E_ALIGN = -6,      /* a pointer is not aligned as the kernels require             */
  QMM_E_WORKSPACE = -7,  /* workspace/scratch missing or smaller than the query says    */
  QMM_E_MODE = -8,       /* unknown zero-point kind or MoE mode                         */
  QMM_E_DEVICE = -9,     /* no usable gfx950 device / library not initialised           */
  QMM_E_PARAM = -10      /* a quantization scale not finite and positive, or a zero
                            point outside the code range                                */
};

/* ---------------------------------------------------------------------------
 * qmm_nbits -- C[M][N] = A[M][K] . dequant(W)^T (+ bias)       ([P1] "What", commit 1)
 *
 *   A        [M][K] of a_type (QMM_F32, QMM_F16, QMM_BF16), contiguous, 16-byte aligned.
 *   W        packed codes, bits in {2, 3, 4, 8} ([P1] kernel unit-test leaves Wu2, Wu3,
 *            Wu4, Wi8; 8 = signed), block in {16, 32, 64, 128, 256} (3 bits: >= 32).
 *   scales   fp16 [N][nblk].
 *   zp       per zp_kind (see above); uniform_zp used only for QMM_ZP_UNIFORM.
 *   bias     [N] of c_type, or NULL.
 *   C        [M][N] of c_type.
 *   workspace, workspace_bytes: device scratch of at least
 *            qmm_nbits_workspace_bytes(M, K, N, a_type) bytes (may be NULL when that is 0).
 * Paths: M <= 8 runs the weight-streaming GEMV, which reads A in its own type
 * and accumulates in fp32.  M > 8 runs a matrix-core path: A is rounded to fp16
 * once into the workspace (rows of K rounded up to a multiple of 64, padded with
 * zeros, for any a_type), each weight is dequantized exactly in fp32 and rounded
 * to fp16, and the products are accumulated in fp32 on the fp16 matrix cores.
 * For 8 < M <= 64 with block >= 32 a skinny kernel (16-row M tiles, each weight
 * loaded once) runs; otherwise 256 x 256 output tiles.  When either grid would
 * not fill the chip, the reduction over K is split into a number of parts fixed
 * by the shape; fp32 partial sums [parts][M][N] follow A in the workspace and are
 * added in part order by a second kernel.
 * ------------------------------------------------------------------------- */
qmm_status qmm_nbits(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                     const uint8_t* W, int bits, int block, const uint16_t* scales,
                     const void* zp, int zp_kind, float uniform_zp, const void* bias,
                     void* C, int c_type, void* workspace, size_t workspace_bytes,
                     void* stream);

size_t qmm_nbits_workspace_bytes(int64_t M, int64_t K, int64_t N, int a_type);

/* Host-only check of qmm_nbits arguments: returns the status qmm_nbits would
 * refuse with (or QMM_OK).  Never dereferences a pointer, needs no GPU. */
qmm_status qmm_validate_nbits(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                              const uint8_t* W, int bits, int block, const uint16_t* scales,
                              const void* zp, int zp_kind, const void* bias, const void* C,
                              int c_type, const void* workspace, size_t workspace_bytes);

/* ---------------------------------------------------------------------------
 * qmm_codebook4 -- C[M][N] = A . (codebook[q] * absmax)^T (+ bias)
 *                                     ([P3] "Summary", "Technical details")
 *   A        [M][K] of a_type (QMM_F16 or QMM_BF16; QMM_F32 also accepted).
 *   W        packed 4-bit codes [N][nblk][block/2], block in {16..256}, power of two.
 *   absmax   fp32 [N][nblk].
 *   codebook fp32 [16] (any values; NF4/FP4 tables are sorted in [-1, 1]).
 *   bias     [N] of c_type, or NULL.   C [M][N] of c_type.
 *   workspace, workspace_bytes: device scratch of at least
 *            qmm_codebook4_workspace_bytes(M, K, N, a_type) bytes (NULL when that is 0).
 *            That size is nonzero from M = 4 on (except M = 4 with N * K <= 2^24).
 *            It is needed for M > 8, and for 4 <= M <= 8 with a 16-bit c_type (the
 *            size does not depend on c_type).
 * Paths: M <= 8 weight-streaming GEMV (fp32 FMA, codebook staged in LDS), except
 * 4 <= M <= 8 with a QMM_F16 or QMM_BF16 output and block >= 32, which takes the
 * skinny kernel below (the GEMV's work grows with M, the skinny kernel's does not up
 * to 16 rows; the fp16 operand rounding is well below the 16-bit output's).  M = 4
 * with N * K <= 2^24 stays on the GEMV (its four-row form is the faster there); the
 * path is a function of the shape and output type only.
 * The matrix-core paths round A to fp16 once into the workspace (as for qmm_nbits)
 * and use weights fp16(fp32(codebook[q] * absmax)): the skinny kernel for M <= 64
 * with block >= 32, 256 x 256 tiles otherwise (as for qmm_nbits).
 * ------------------------------------------------------------------------- */
qmm_status qmm_codebook4(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                         const uint8_t* W, int block, const float* absmax,
                         const float* codebook, const void* bias, void* C, int c_type,
                         void* workspace, size_t workspace_bytes, void* stream);

size_t qmm_codebook4_workspace_bytes(int64_t M, int64_t K, int64_t N, int a_type);

qmm_status qmm_validate_codebook4(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                                  const uint8_t* W, int block, const float* absmax,
                                  const float* codebook, const void* bias, const void* C,
                                  int c_type, const void* workspace, size_t workspace_bytes);

/* ---------------------------------------------------------------------------
 * Nested (double-quantized) absmax for the codebook format ([P3] "Testing plan":
 * nested and non-nested absmax).  Block i (flat index n * nblk + b) stores an 8-bit
 * code into a 256-entry fp32 table; `group` consecutive blocks share one fp32 scale,
 * and one fp32 offset is added back:
 *   absmax_i = fp32(fp32(table[codes[i]] * scales[i / group]) + offset)
 * ------------------------------------------------------------------------- */
typedef struct {
  const uint8_t* codes;  /* uint8 [N][nblk] (device)                          */
  const float* table;    /* fp32 [256] (device)                               */
  const float* scales;   /* fp32 [ceil(N * nblk / group)] (device)            */
  float offset;
  int group;             /* blocks per scale, >= 1 (bitsandbytes uses 256)    */
} qmm_nested_absmax;

/* out[i] = absmax_i for i < count (fp32, device); `absmax` is a HOST pointer to the
 * descriptor.  Bit-exact with the definition above. */
qmm_status qmm_dequantize_absmax_nested(const qmm_nested_absmax* absmax, int64_t count, float* out,
                                        void* stream);

/* qmm_codebook4 with nested absmax: the absmax of the N * nblk blocks is decoded once
 * into the workspace (one small launch), then qmm_codebook4 runs on it, so results
 * are those of qmm_codebook4 on the decoded values.  workspace: at least
 * qmm_codebook4_nested_workspace_bytes(M, K, N, a_type, block) bytes, 256-byte
 * aligned (the decoded absmax first, then qmm_codebook4's workspace). */
qmm_status qmm_codebook4_nested(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                                const uint8_t* W, int block, const qmm_nested_absmax* absmax,
                                const float* codebook, const void* bias, void* C, int c_type,
                                void* workspace, size_t workspace_bytes, void* stream);
size_t qmm_codebook4_nested_workspace_bytes(int64_t M, int64_t K, int64_t N, int a_type, int block);

/* ---------------------------------------------------------------------------
 * qmm_fp16_uniform_value -- is every fp16 zero point bitwise equal?
 *                                     ([P1] "What", commit 1: detected once per buffer)
 *   zp       fp16 [count] (device).
 *   scratch  device buffer of at least qmm_uniform_scratch_bytes() bytes.
 *   is_uniform, value: HOST pointers receiving the flag and the fp32 value.
 * A NaN first element is never uniform; count == 0 is not uniform.
 * Synchronizes `stream` (call once per weight buffer, not per matmul).
 * ------------------------------------------------------------------------- */
qmm_status qmm_fp16_uniform_value(const uint16_t* zp, int64_t count, void* scratch,
                                  size_t scratch_bytes, int* is_uniform, float* value,
                                  void* stream);
size_t qmm_uniform_scratch_bytes(void);

/* ---------------------------------------------------------------------------
 * Dequantize to a dense matrix out[N][K] (out_type QMM_F32 or QMM_F16).
 * Bit-exact with the definitions above (fp16 output is the RNE rounding of the
 * fp32 weight, i.e. the operand the matrix-core paths use).
 * ------------------------------------------------------------------------- */
qmm_status qmm_dequantize_nbits(const uint8_t* W, int bits, int block, const uint16_t* scales,
                                const void* zp, int zp_kind, float uniform_zp, int64_t N,
                                int64_t K, void* out, int out_type, void* stream);

qmm_status qmm_dequantize_codebook4(const uint8_t* W, int block, const float* absmax,
                                    const float* codebook, int64_t N, int64_t K, void* out,
                                    int out_type, void* stream);

/* ---------------------------------------------------------------------------
 * qmoe_decode_fused -- top-k MoE decode with u4 expert weights.
 *                                     ([P2] "Summary", "Why", "What")
 * For token t in [0,T) and slot j in [0,k) with expert e = expert_ids[t][j]:
 *   [g ; u] = W1_e . x'_t + b1_e     (fc1: 2I outputs, g = rows [0,I), u = rows [I,2I))
 *   h       = fp16(g * sigmoid(g) * u)
 *   z       = W2_e . h' + b2_e       (fc2: H outputs)
 *   Y[t]    = fp16( sum over j = 0..k-1 in order of expert_w[t][j] * z )
 * QMOE_FP: x' = x, h' = h.  QMOE_INT8_ACT: x' and h' are symmetric int8 per 32
 * consecutive values (scale fp32(amax/127), codes rint(fp32(v*fp32(127/amax))))
 * and the products with (q - zp) are summed exactly in int32 per 32 values.
 *
 *   X          fp16 [T][H]            Y fp16 [T][H]
 *   expert_ids int32 [T][k], each in [0, E)  (an id outside is clamped into it on device)
 *   expert_w   fp32 [T][k]
 *   fc1.W      uint8 [E][2I][nblk(H)][block/2]   fc1.scales fp16 [E][2I][nblk(H)]
 *   fc1.zp     uint8 [E][2I][ceil(nblk(H)/2)] packed u4, or NULL (zp = 8)
 *   fc1.bias   fp16 [E][2I] or NULL
 *   fc2.*      the same with [E][H][..] over K = I
 *   bits       4.  block in {32, 64, 128, 256} (int8 mode additionally needs
 *              H % 32 == 0 and I % 32 == 0).
 *   scratch    device buffer of at least qmoe_decode_scratch_bytes(T, H, I, k, mode),
 *              256-byte aligned.  Layout (each region at a 256-byte boundary): the
 *              sync words of the single-launch form in the first 8448 bytes (the same
 *              place for every shape and mode): uint32 [0] top arrival count, [2] error
 *              flag, then in each of the next 32 256-byte slots an arrival sub-counter
 *              and a phase word; then fp16 h [T][k][I] at offset 8448, then in
 *              int8 mode int8 x codes [T][H], fp32 x scales [T][H/32], int8 h codes
 *              [T][k][I], fp32 h scales [T][k][I/32].  The sync words must be zero
 *              before the first call on a buffer (zero the whole buffer once, e.g.
 *              hipMemset); every call leaves the counters zero again and the phases
 *              equal, at 0 or 1.  The error flag is set, and left set, by a call whose wait inside
 *              the launch gave up after 1 s (its output is then invalid).  Calls that
 *              share a scratch buffer must not overlap.
 *   Launches   one launch of all of it by default: a grid that is resident all at
 *              once (its size is the kernel's occupancy times the compute units) runs
 *              its fc1 share, publishes h, waits for every work-group's h and streams
 *              its fc2 share (first loads issued before the wait; int8 mode: each
 *              work-group quantizes h itself).  The two-kernel form (fc1 + SwiGLU,
 *              then fc2 + combine; int8 mode adds the h quantizer between them) runs
 *              instead where the up-front timing finds it more than 5% faster, or
 *              where no single-launch plan fits.  The one-launch form
 *              needs the compute units to itself for that wait: a kernel on another
 *              stream that holds them for more than 1 s makes the wait give up (error
 *              flag above; the call's Y is then filled with fp16 NaN and
 *              qmoe_decode_status reports it).  Every form gives the same bits.
 *   E          num_experts: the first call of a shape times tiling candidates on
 *              other expert sets, writing only scratch.
 * ------------------------------------------------------------------------- */
typedef struct {
  const uint8_t* W;
  const uint16_t* scales;
  const uint8_t* zp;    /* packed u4 or NULL */
  const uint16_t* bias; /* fp16 or NULL */
} qmoe_weights;

qmm_status qmoe_decode_fused(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E,
                             int k, const int32_t* expert_ids, const float* expert_w,
                             qmoe_weights fc1, qmoe_weights fc2, int bits, int block,
                             int mode, uint16_t* Y, void* scratch, size_t scratch_bytes,
                             void* stream);

size_t qmoe_decode_scratch_bytes(int64_t T, int64_t H, int64_t I, int k, int mode);

/* ---------------------------------------------------------------------------
 * qmoe_ragged_mm -- the expert matmul of a multi-token MoE burst ([P1]/[P2] "Kernel Unit
 * Test Results": qmoe_ragged_mm, leaf Xfp16_Wu4_Yfp16; [P2] "Related issue or design":
 * T-token bursts through the QMoE layer).
 *   Rows of X are grouped by expert: expert e owns rows row_offsets[e] ..
 *   row_offsets[e+1] - 1 (row_offsets [E+1] int32 on the device, nondecreasing,
 *   row_offsets[0] = 0, row_offsets[E] = R; values are clamped into [0, R] on the
 *   device, and rows no expert owns are not written).  For each such row r
 *     Y[r] = fp16( X[r] . W16_e^T + bias_e )
 *   with W16_e = fp16 of the exact dequantized u4 weight (w = fp32(fp32(q - zp) * s),
 *   zp 8 when w.zp is NULL) and the products accumulated in fp32 on the fp16 matrix
 *   cores (the operand rounding of the matrix-core paths of qmm_nbits).
 *   X      fp16 [R][K], 16-byte aligned, K a multiple of 8.
 *   w      W [E][N][nblk][block/2], scales fp16 [E][N][nblk], zp packed u4
 *          [E][N][ceil(nblk/2)] or NULL, bias fp16 [E][N] or NULL.
 *   bits   4.  block: power of two in [32, 256].   Y fp16 [R][N].
 *   One launch; tiles of 16 to 64 rows of one expert per work-group.
 * ------------------------------------------------------------------------- */
qmm_status qmoe_ragged_mm(const uint16_t* X, int64_t R, int64_t K, int64_t N, int64_t E,
                          const int32_t* row_offsets, qmoe_weights w, int bits, int block,
                          uint16_t* Y, void* stream);

/* qmoe_decode_fused_noalloc -- qmoe_decode_fused for callers that cannot allocate
 * (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments and results as qmoe_decode_fused, without scratch: the scratch is a
 * static device array of QMOE_NOALLOC_SCRATCH_BYTES inside the library, one per
 * device, held until the process ends.  A shape that needs more
 * (qmoe_decode_scratch_bytes) is refused with QMM_E_WORKSPACE.  The call never times
 * tiling candidates: it uses the choice an earlier qmoe_decode_fused call made for the
 * shape, else the default tiling, and so calls no allocating routine.  All calls on
 * one device share the array: calls that overlap on one device (other streams, other
 * threads) race and must not be made. */
#define QMOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
qmm_status qmoe_decode_fused_noalloc(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E,
                                     int k, const int32_t* expert_ids, const float* expert_w,
                                     qmoe_weights fc1, qmoe_weights fc2, int bits, int block, int mode,
                                     uint16_t* Y, void* stream);

/* qmoe_decode_status -- whether a single-launch qmoe_decode_fused call on this scratch
 * buffer gave up its wait ([P2] "What": a call must not report an error it did not
 * cause, nor hide one it did).  Reads the error word of the scratch layout above into
 * *timed_out (HOST pointer: 1 = some call gave up, its Y was filled with fp16 NaN;
 * 0 = none), then clears it.  T, H, I, k, mode: those of the calls made on the buffer.
 * Synchronizes `stream`.  Returns
 * QMM_E_NULL / QMM_E_WORKSPACE / QMM_E_ALIGN for a missing, short or misaligned buffer,
 * or the hipError_t of the copy. */
qmm_status qmoe_decode_status(void* scratch, size_t scratch_bytes, int64_t T, int64_t H, int64_t I,
                              int k, int mode, int* timed_out, void* stream);

qmm_status qmm_validate_qmoe(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E,
                             int k, const int32_t* expert_ids, const float* expert_w,
                             qmoe_weights fc1, qmoe_weights fc2, int bits, int block, int mode,
                             const uint16_t* Y, const void* scratch, size_t scratch_bytes);

/* ---------------------------------------------------------------------------
 * Activation quantize / dequantize and the fused quantized SwiGLU
 *                       ([P1] "Why": the per-layer chain Q(gate) -> qsigmoid -> 2x qmul ->
 *                        Q(up) -> DQ; "What", commit 4: fused Q -> DQ round trip and
 *                        fused quantized SwiGLU, each exactly equal to the unfused chain)
 *
 * Per-tensor parameters (scale, zero_point); codes are uint8 (bits = 8) or uint16
 * (bits = 16).  Element by element:
 *   Q(x)    = min(max(rint(fp32(x / scale)) + zero_point, 0), 2^bits - 1)
 *             (ties to even, the quotient correctly rounded; a NaN quotient gives 0)
 *   DQ(q)   = fp32((q - zero_point) * scale)
 *   sigmoid = the fp32 rounding of 1 / (1 + e^-v), evaluated in fp64
 * x, y: [n] of x_type / y_type (QMM_F32, QMM_F16, QMM_BF16; 16-bit outputs are the
 * nearest value of the fp32 result).  Device pointers, element-aligned; codes
 * 2-byte aligned for bits = 16.  scale must be finite and > 0, zero_point in
 * [0, 2^bits - 1] (else QMM_E_PARAM); bits other than 8 and 16 give QMM_E_BITS.
 * n = 0 launches nothing.  The fused ops give the bits of the unfused chain.
 * ------------------------------------------------------------------------- */
typedef struct {
  float scale;
  int32_t zero_point;
} qmm_qparams;

qmm_status qmm_quantize_linear(const void* x, int x_type, int64_t n, qmm_qparams q, int bits,
                               void* codes, void* stream);
qmm_status qmm_dequantize_linear(const void* codes, int64_t n, qmm_qparams q, int bits, void* y,
                                 int y_type, void* stream);
/* y = DQ(Q(x)), y of x_type: one launch, no code tensor. */
qmm_status qmm_fake_quantize(const void* x, int x_type, int64_t n, qmm_qparams q, int bits,
                             void* y, void* stream);
/* codes_out = Q(sigmoid(DQ(codes_in; in)); out). */
qmm_status qmm_qsigmoid(const void* codes_in, int64_t n, qmm_qparams in, qmm_qparams out, int bits,
                        void* codes_out, void* stream);
/* c = Q(fp32(DQ(a; qa) * DQ(b; qb)); qc). */
qmm_status qmm_qmul(const void* a, qmm_qparams qa, const void* b, qmm_qparams qb, int64_t n,
                    qmm_qparams qc, int bits, void* c, void* stream);
/* The quantized SwiGLU chain in one launch, y of x_type:
 *   g = Q(gate; q[0]);  t = qsigmoid(g -> q[1]);  m = qmul(g, t -> q[2]);
 *   u = Q(up; q[3]);    h = qmul(m, u -> q[4]);   y = DQ(h; q[4]).
 * q: HOST array of five parameter pairs (gate, sigmoid, silu, up, out). */
qmm_status qmm_qswiglu(const void* gate, const void* up, int x_type, int64_t n, int bits,
                       const qmm_qparams* q, void* y, void* stream);

/* ---------------------------------------------------------------------------
 * Tuning control and introspection.
 * qmm_tuning_mode: 0 = time candidates on the first call of a shape (default),
 *   1 = never time, always use the default tiling, 2 = force candidate
 *   `forced_index` (for tests: every candidate must give identical bits).
 * qmm_tuned_choice: the candidate index chosen for the last call of the given
 *   entry (0 = qmm_nbits GEMV, 1 = qmm_codebook4 GEMV, 2 = qmoe fc1, 3 = qmoe fc2,
 *   4 = qmoe single-launch form, -1 when the last MoE call used two kernels), or -1
 *   if none; qmm_num_candidates gives the candidate count per entry.  Forced MoE
 *   indices below n(2) * n(3) pick the two-kernel form (fc1 = index % n(2),
 *   fc2 = index / n(2)); index n(2) * n(3) + c picks candidate c of entry 4.
 * qmm_clear_tuning forgets every cached choice.
 * ------------------------------------------------------------------------- */
qmm_status qmm_set_tuning(int mode, int forced_index);
int qmm_num_candidates(int entry);
int qmm_tuned_choice(int entry);
void qmm_clear_tuning(void);

/* GEMV candidates of entries 0 and 1: indices 0, 1, 2 are the v_dot8 / fp32 kernels
 * with 1, 2, 4 weight rows per lane; 3 is the matrix-core form of the 2-bit GEMV
 * (v_mfma_scale_f32_16x16x128_f8f6f4: the activation digit planes as e4m3 rows, the
 * codes as e2m1 nibbles, every product and sum exact; 16 weight rows per wave).  All
 * four give the same bits.  Where the matrix-core form does not serve a shape, index 3
 * runs the v_dot8 kernel with 2 rows per lane and the up-front timing skips it.
 * qmm_nbits_gemv_matrix_core_form: 1 when qmm_nbits at this shape (16-byte aligned
 * W, A and scales) has the matrix-core form among its candidates: bits = 2, M = 1,
 * block = 64 with ceil(K / 64) a multiple of 8, the activations' operand (4 KiB per
 * 256 codes) within LDS, and the lanes-per-row split of the v_dot8 kernel (fixed by K
 * and N) of 16 or 32 lanes, with ceil(K / 256) a multiple of a quarter of it; else 0. */
int qmm_nbits_gemv_matrix_core_form(int64_t M, int64_t K, int64_t N, int bits, int block);

/* The selection rule of the up-front timing, exposed for host-only checks:
 * times_us[r * ncand + c] is round r of candidate c; round 0 is discarded, the
 * least total over rounds 1..rounds-1 wins, ties go to the lower index.
 * Returns -1 for bad arguments. */
int qmm_tuner_pick(const double* times_us, int rounds, int ncand);

/* The MoE decode's choice between its single-launch forms and the two-kernel pair,
 * exposed for host-only checks: candidates 0 .. ncand-2 are single-launch forms and
 * candidate ncand-1 the pair, totals as in qmm_tuner_pick.  The fastest single launch
 * is chosen unless the pair's total is more than 5% below it (ties to the lower
 * index).  Returns -1 for bad arguments (ncand < 2 or rounds < 2). */
int qmm_tuner_pick_single_launch(const double* times_us, int rounds, int ncand);

/* ---------------------------------------------------------------------------
 * Measurement helper (not part of the computation): reads `bytes` of device memory
 * (16-byte aligned, a multiple of 16) once with 128-bit loads, `groups` work-groups of
 * 256 threads each reading one contiguous range, and writes the xor of what each
 * work-group read to sink[group] (uint32 [groups], device).  Timing it gives the HBM
 * read rate a plain streaming kernel reaches, the practical ceiling of the weight-
 * streaming kernels.  groups in [1, 2^20].
 * ------------------------------------------------------------------------- */
qmm_status qmm_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int groups, void* stream);

/* Measurement helpers (not part of the computation): kernel execution times.
 * qmm_launch_timing_begin(n): from now on, the first n kernel launches that the library
 * makes from the calling host thread each record the start and the end of their execution
 * on the device (hipExtLaunchKernel with a pair of HIP events, created here on the current
 * device); the launches themselves are unchanged.  n in [1, 65536]; QMM_E_MODE if timing
 * is already on for this thread.  Do not switch it on around stream capture.
 * qmm_launch_timing_end(us, n_max, count): switches it off, waits for the recorded
 * launches, writes the duration in microseconds of each (launch order) to us[0..] (HOST
 * array, at most n_max values), the number of timed launches to *count (HOST), and frees
 * the events.  With timing off it writes *count = 0. */
qmm_status qmm_launch_timing_begin(int n);
qmm_status qmm_launch_timing_end(float* us, int n_max, int* count);

/* Human-readable name of a status code (static storage). */
const char* qmm_status_string(qmm_status s);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
