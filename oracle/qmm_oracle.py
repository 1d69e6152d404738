"""Oracle for the fused low-bit dequantize-matmul path: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module.  It shares no code with the HIP library and
imports nothing from it.

Sources (cited by page and section):
  [P1] hip-ep pull request 1318, "bits=2 MatMulNBits" (2-bit phi4-14B on gfx1151):
       sections "Why" and "What" (commit 1: u2 GEMV/WMMA templated on A/C types,
       A cast to fp16 once for the prefill tiles, uniform fp16 zero point becomes a
       scalar; commit 4: fused Q->DQ round trip exactly equal to the unfused chain),
       section "Performance" (model: MatMulNBits bits=2, block 64, fp16 zero
       points all 1.5, fp32 activations).
  [P2] hip-ep pull request 1328, "fused QMoE decode picks tiling up front":
       sections "Summary", "Why", "What" (fc1 -> SwiGLU -> fc2 per token over the
       top-k experts; dp4a variant with int8 activations; CPU reference that
       rounds and quantizes where the kernels do).
  [P3] bitsandbytes pull request 1979, "[ROCm] Fused 4-bit SIMT GEMM":
       sections "Summary" and "Technical details" (NF4/FP4 16-entry centroids,
       per-block absmax, scale applied per chunk).

Every function is the plain definition of its result, accumulated in fp64.  The
readings taken where the pages are silent are listed in the design notes and
restated at each function:
  * codes are packed LSB-first along K inside each byte, row layout
    [N][nblk][B*bits/8], ragged last block padded (padding never read);
  * dequant is w = fp32(fp32(q - zp) * fp32(scale)), each step one rounding;
  * codebook dequant is w = fp32(codebook[q] * absmax);
  * the zero point defaults to 2^(bits-1) when absent;
  * SwiGLU splits the fc1 output as g = rows [0, I), u = rows [I, 2I) and
    computes h = g * sigmoid(g) * u, stored as fp16;
  * int8 activations are symmetric, one fp32 scale per 32 consecutive values.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(brute force with exact rationals, closed forms, invariants, library routines).
"""
from __future__ import annotations

import numpy as np

# zero-point kinds, by name
ZP_NONE, ZP_PACKED, ZP_F16, ZP_UNIFORM = "none", "packed", "f16", "uniform"


# ---------------------------------------------------------------------------
# Rounding primitives
# ---------------------------------------------------------------------------

def to_f32(x) -> np.ndarray:
    """Round fp64 values to the nearest fp32 (ties to even): numpy's cast."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def to_f16(x) -> np.ndarray:
    """Round fp64 values to the nearest fp16 (ties to even): numpy's cast."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 is the top half of an fp32: widen the bit pattern."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bits.

    Written on the integer bit pattern: add half an ulp of the kept part
    (0x7fff, plus one when the kept part is odd), then drop the low 16 bits.
    NaN keeps its sign and becomes a quiet NaN.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = np.isnan(np.asarray(x, dtype=np.float32))
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan_bits = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    return np.where(is_nan, nan_bits, r).astype(np.uint16)


def to_bf16_f64(x) -> np.ndarray:
    """fp32 -> nearest bf16, returned as fp64 values."""
    return bf16_bits_to_f64(f32_to_bf16_bits(x))


def activations_f64(A, a_dtype: str) -> np.ndarray:
    """Activation storage (fp32 array, or fp16/bf16 bit patterns) -> fp64 values."""
    if a_dtype == "f32":
        return np.asarray(A, dtype=np.float32).astype(np.float64)
    if a_dtype == "f16":
        return f16_bits_to_f64(A)
    if a_dtype == "bf16":
        return bf16_bits_to_f64(A)
    raise ValueError(a_dtype)


# ---------------------------------------------------------------------------
# Unpacking and dequantization  ([P1] "What", commit 1; [P3] "Summary")
# ---------------------------------------------------------------------------

def _field(lo, hi, shift, bits: int) -> np.ndarray:
    """The `bits`-wide field at bit `shift` of the 16-bit little-endian pair (lo, hi)."""
    v = lo.astype(np.uint16) | (hi.astype(np.uint16) << np.uint16(8))
    return ((v >> np.asarray(shift, dtype=np.uint16)) & np.uint16((1 << bits) - 1)).astype(np.uint8)


def unpack_codes(W, bits: int, K: int, block: int) -> np.ndarray:
    """Codes q[n, k] from packed W[N][nblk][block*bits/8].

    Element k sits in block b = k // block at position j = k % block; its code is the
    `bits`-wide field starting at bit j*bits of the block's little-endian bit stream
    (bit i of byte n of the block is stream bit 8n + i; least significant field first,
    so a 3-bit field may continue into the next byte).  bits = 2, 3, 4: unsigned codes.
    bits = 8: the byte is a signed two's-complement code in [-128, 127].  Codes past K
    are not read.
    """
    W = np.asarray(W, dtype=np.uint8)
    k = np.arange(K)
    b = k // block
    j = k % block
    if bits == 8:
        return W[..., b, j].view(np.int8)
    nbytes = W.shape[-1]
    pos = j * bits
    byte = pos // 8
    lo = W[..., b, byte]
    hi = np.where(byte + 1 < nbytes, W[..., b, np.minimum(byte + 1, nbytes - 1)], 0)
    return _field(lo, hi, pos % 8, bits)


def unpack_zero_points(zp_packed, bits: int, nblk: int) -> np.ndarray:
    """Packed per-block zero points zp[n][ceil(nblk*bits/8)] -> [N, nblk].

    Same field order as the weights: block b is the field at bit b*bits of the row's
    bit stream.  bits = 8: signed bytes."""
    zp_packed = np.asarray(zp_packed, dtype=np.uint8)
    b = np.arange(nblk)
    if bits == 8:
        return zp_packed[..., b].view(np.int8)
    nbytes = zp_packed.shape[-1]
    pos = b * bits
    byte = pos // 8
    lo = zp_packed[..., byte]
    hi = np.where(byte + 1 < nbytes, zp_packed[..., np.minimum(byte + 1, nbytes - 1)], 0)
    return _field(lo, hi, pos % 8, bits)


def default_zero_point(bits: int) -> float:
    """Zero point when none is given: 2^(bits-1) for unsigned codes, 0 for signed int8."""
    return 0.0 if bits == 8 else float(1 << (bits - 1))


def zero_points_f64(zp, zp_kind: str, bits: int, N: int, nblk: int,
                    uniform_zp: float = 0.0) -> np.ndarray:
    """Per-(row, block) zero point as fp64 [N, nblk] for each zero-point kind.

    none -> default_zero_point(bits); packed -> the code (signed for bits = 8);
    f16 -> the fp16 value; uniform -> the scalar (given as fp32).
    """
    if zp_kind == ZP_NONE:
        return np.full((N, nblk), default_zero_point(bits))
    if zp_kind == ZP_PACKED:
        return unpack_zero_points(zp, bits, nblk).astype(np.float64)
    if zp_kind == ZP_F16:
        return f16_bits_to_f64(zp).reshape(N, nblk)
    if zp_kind == ZP_UNIFORM:
        return np.full((N, nblk), float(np.float32(uniform_zp)))
    raise ValueError(zp_kind)


def dequant_nbits(W, bits, K, block, scales_f16, zp=None, zp_kind=ZP_NONE,
                  uniform_zp=0.0) -> np.ndarray:
    """Dequantized fp32 weights [N, K]: w = fp32(fp32(q - zp) * scale).

    The subtraction and the multiplication are each one fp32 rounding of the
    exact result (fp32 products are exact in fp64, so rounding the fp64 product
    once is the fp32 multiply).
    """
    q = unpack_codes(W, bits, K, block).astype(np.float64)
    N = q.shape[0]
    nblk = (K + block - 1) // block
    z = zero_points_f64(zp, zp_kind, bits, N, nblk, uniform_zp)
    s = f16_bits_to_f64(scales_f16).reshape(N, nblk)
    blk = np.arange(K) // block
    d = to_f32(q - z[:, blk]).astype(np.float64)
    return to_f32(d * s[:, blk])


def nested_absmax(codes, table, scales, offset, group: int) -> np.ndarray:
    """Per-block absmax stored double-quantized ([P3] "Testing plan": nested absmax):
    block i (the flat index n * nblk + b) has an 8-bit code c_i into a 256-entry fp32
    table, one fp32 scale per `group` consecutive blocks, and one fp32 offset:

        absmax_i = fp32(fp32(table[c_i] * scales[i // group]) + offset)

    (each operation one fp32 rounding of its exact result).  Returns fp32 with the
    shape of `codes`."""
    c = np.asarray(codes, dtype=np.uint8)
    t = np.asarray(table, dtype=np.float32).astype(np.float64)
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    i = np.arange(c.size).reshape(c.shape)
    prod = to_f32(t[c] * sc[i // group]).astype(np.float64)
    return to_f32(prod + float(np.float32(offset)))


def dequant_codebook4(W, K, block, absmax, codebook) -> np.ndarray:
    """Dequantized fp32 weights [N, K]: w = fp32(codebook[q] * absmax[n, block])."""
    q = unpack_codes(W, 4, K, block)
    cb = np.asarray(codebook, dtype=np.float32).astype(np.float64)
    N = q.shape[0]
    nblk = (K + block - 1) // block
    am = np.asarray(absmax, dtype=np.float32).astype(np.float64).reshape(N, nblk)
    blk = np.arange(K) // block
    return to_f32(cb[q] * am[:, blk])


# ---------------------------------------------------------------------------
# Matmuls  ([P1] "What", commit 1; [P3] "Summary", "Technical details")
# ---------------------------------------------------------------------------

def row_prescale_exponents(a64) -> np.ndarray:
    """Per-row power-of-two pre-scale of the matrix-core activation cast.

    For row m with largest magnitude |a| = f * 2^E (f in [0.5, 1)), the row is
    multiplied by 2^s with s = min(15 - E, 126) before its fp16 rounding, which
    puts the largest magnitude in [2^14, 2^15) (the cap keeps 2^-s a normal fp32
    for rows of tiny values): no value overflows fp16 and the small values keep
    their bits.  A row that is all zero, or whose largest magnitude is not finite,
    is not scaled (exponent 0).  Returns the exponents s as int64 [M].
    """
    a = np.asarray(a64, dtype=np.float64)
    amax = np.max(np.abs(a), axis=-1) if a.shape[-1] > 0 else np.zeros(a.shape[:-1])
    out = np.zeros(amax.shape, dtype=np.int64)
    ok = np.isfinite(amax) & (amax > 0)
    _, E = np.frexp(np.where(ok, amax, 1.0))
    out[ok] = np.minimum(15 - E[ok], 126)
    return out


def _round_operand(x64, mode):
    """Declared operand rounding of a path that feeds 16-bit matrix cores.

    "f16": nearest fp16 of each value.  "bf16": nearest bf16 of the fp32 value.
    "f16_rows": the activation cast of the matrix-core paths: each row m is scaled
    by 2^s_m (row_prescale_exponents), rounded to the nearest fp16 and scaled back,
    a' = fp16(a * 2^s_m) * 2^-s_m (both scalings are exact).
    """
    if mode is None:
        return x64
    if mode == "f16":
        return to_f16(x64).astype(np.float64)
    if mode == "bf16":
        return to_bf16_f64(to_f32(x64))
    if mode == "f16_rows":
        x = np.asarray(x64, dtype=np.float64)
        s = row_prescale_exponents(x)[..., None].astype(np.int32)
        return np.ldexp(to_f16(np.ldexp(x, s)).astype(np.float64), -s)
    raise ValueError(mode)


def matmul_f64(a64, w64, bias64=None) -> np.ndarray:
    """y[m, n] = sum_k a[m, k] * w[n, k] (+ bias[n]) in fp64."""
    y = a64 @ w64.T
    if bias64 is not None:
        y = y + bias64[None, :]
    return y


def qmm_nbits(A, a_dtype, W, bits, K, block, scales_f16, zp=None, zp_kind=ZP_NONE,
              uniform_zp=0.0, bias=None, bias_dtype="f32", a_round=None, w_round=None,
              rows=None) -> np.ndarray:
    """MatMulNBits: y = A . dequant(W)^T (+ bias), fp64, unrounded output.

    a_round / w_round name a declared rounding of the operands (e.g. "f16" for a
    path that casts A to fp16 once and dequantizes W tiles to fp16).  `rows`
    restricts the computation to a subset of output columns n (for sampling).
    """
    W = np.asarray(W)
    scales_f16 = np.asarray(scales_f16)
    if rows is not None:
        rows = np.asarray(rows)
        W = W[rows]
        scales_f16 = scales_f16[rows]
        if zp is not None and zp_kind in (ZP_PACKED, ZP_F16):
            zp = np.asarray(zp)[rows]
        if bias is not None:
            bias = np.asarray(bias)[rows]
    w = dequant_nbits(W, bits, K, block, scales_f16, zp, zp_kind, uniform_zp)
    a = activations_f64(A, a_dtype)
    b = None if bias is None else activations_f64(bias, bias_dtype)
    return matmul_f64(_round_operand(a, a_round), _round_operand(w.astype(np.float64), w_round), b)


def qmm_codebook4(A, a_dtype, W, K, block, absmax, codebook, bias=None, a_round=None,
                  w_round=None, rows=None) -> np.ndarray:
    """Codebook 4-bit matmul: y = A . (codebook[q] * absmax)^T (+ bias), fp64."""
    W = np.asarray(W)
    absmax = np.asarray(absmax)
    if rows is not None:
        rows = np.asarray(rows)
        W, absmax = W[rows], absmax[rows]
        if bias is not None:
            bias = np.asarray(bias)[rows]
    w = dequant_codebook4(W, K, block, absmax, codebook)
    a = activations_f64(A, a_dtype)
    b = None if bias is None else activations_f64(bias, a_dtype)
    return matmul_f64(_round_operand(a, a_round), _round_operand(w.astype(np.float64), w_round), b)


# ---------------------------------------------------------------------------
# Uniform zero point  ([P1] "What", commit 1: all-equal fp16 tensor -> scalar)
# ---------------------------------------------------------------------------

def fp16_uniform_value(zp_f16_bits):
    """(is_uniform, value): every fp16 bit pattern equal to the first and not NaN."""
    z = np.asarray(zp_f16_bits, dtype=np.uint16).ravel()
    if z.size == 0:
        return False, 0.0
    first = z[0]
    if np.isnan(np.uint16(first).view(np.float16)):
        return False, 0.0
    if np.all(z == first):
        return True, float(np.uint16(first).view(np.float16))
    return False, 0.0


# ---------------------------------------------------------------------------
# Int8 activations  ([P2] "Summary"/"Why": dp4a variant with int8 activations)
# ---------------------------------------------------------------------------

def quantize_int8_groups(v64, group: int = 32):
    """Symmetric int8 quantization of each run of `group` values along the last axis.

    amax = max |v|; a zero group gives codes 0 and scale 0.  Otherwise
    inv = fp32(127 / amax), t = fp32(v * inv), q = round-half-even(t) clamped to
    [-127, 127], scale = fp32(amax / 127).  Returns (codes int8, scales fp32).
    """
    v = np.asarray(v64, dtype=np.float64)
    n = v.shape[-1]
    assert n % group == 0
    g = v.reshape(v.shape[:-1] + (n // group, group))
    amax = np.abs(g).max(axis=-1)
    safe = np.where(amax == 0.0, 1.0, amax)
    inv = to_f32(127.0 / safe).astype(np.float64)
    t = to_f32(g * inv[..., None]).astype(np.float64)
    q = np.clip(np.rint(t), -127, 127)
    q = np.where(amax[..., None] == 0.0, 0.0, q)
    s = np.where(amax == 0.0, 0.0, to_f32(safe / 127.0).astype(np.float64))
    return q.reshape(v.shape).astype(np.int8), to_f32(s)


def dequantize_int8_groups(q, s, group: int = 32) -> np.ndarray:
    q64 = np.asarray(q, dtype=np.float64)
    n = q64.shape[-1]
    s64 = np.repeat(np.asarray(s, dtype=np.float32).astype(np.float64), group, axis=-1)
    return q64 * s64.reshape(q64.shape[:-1] + (n,))


# ---------------------------------------------------------------------------
# Fused MoE decode  ([P2] "Summary", "What"; SwiGLU chain from [P1] "Why")
# ---------------------------------------------------------------------------

def sigmoid(x64):
    return 1.0 / (1.0 + np.exp(-x64))


def swiglu(gu64, I: int) -> np.ndarray:
    """h = g * sigmoid(g) * u with g = gu[..., :I], u = gu[..., I:2I] (fp64)."""
    g = gu64[..., :I]
    u = gu64[..., I:2 * I]
    return g * sigmoid(g) * u


def _expert_dequant(fc, e, bits, K, block, N):
    W = np.asarray(fc["W"])[e]
    s = np.asarray(fc["scales"])[e]
    if fc.get("zp") is not None:
        return dequant_nbits(W, bits, K, block, s, np.asarray(fc["zp"])[e], ZP_PACKED)
    return dequant_nbits(W, bits, K, block, s, None, ZP_NONE)


def qmoe_decode(X_f16, ids, rw, fc1, fc2, H, I, block, bits=4, mode="fp"):
    """Top-k MoE decode: for each token t and slot j (expert e = ids[t, j]):

        [g; u] = W1_e . x' + b1_e          (fc1, 2I outputs)
        h      = fp16(g * sigmoid(g) * u)  (SwiGLU, stored as fp16)
        z      = W2_e . h' + b2_e          (fc2, H outputs)
        y_t    = sum_j rw[t, j] * z        (slot order j = 0..k-1)

    mode "fp": x' = x, h' = h.  mode "int8": x' and h' are their symmetric int8
    per-32 quantized-then-dequantized values (quantize_int8_groups).
    Returns fp64 y [T, H] (unrounded).
    """
    X = f16_bits_to_f64(X_f16)
    T = X.shape[0]
    k = ids.shape[1]
    y = np.zeros((T, H))
    cache = {}
    for t in range(T):
        x = X[t]
        if mode == "int8":
            xq, xs = quantize_int8_groups(x)
            x = dequantize_int8_groups(xq, xs)
        for j in range(k):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = (_expert_dequant(fc1, e, bits, H, block, 2 * I).astype(np.float64),
                            _expert_dequant(fc2, e, bits, I, block, H).astype(np.float64))
            w1, w2 = cache[e]
            gu = w1 @ x
            if fc1.get("bias") is not None:
                gu = gu + f16_bits_to_f64(np.asarray(fc1["bias"])[e])
            h = to_f16(swiglu(gu, I)).astype(np.float64)
            if mode == "int8":
                hq, hs = quantize_int8_groups(h)
                h = dequantize_int8_groups(hq, hs)
            z = w2 @ h
            if fc2.get("bias") is not None:
                z = z + f16_bits_to_f64(np.asarray(fc2["bias"])[e])
            y[t] += float(np.float32(rw[t, j])) * z
    return y


# ---------------------------------------------------------------------------
# Ragged multi-token MoE matmul  ([P1]/[P2] "Kernel Unit Test Results": the
# qmoe_ragged_mm leaf Xfp16_Wu4_Yfp16; [P2] "Related issue or design": bursts of
# T tokens through the QMoE layer)
# ---------------------------------------------------------------------------

def group_by_expert(ids, E: int):
    """Rows of a ragged expert batch from top-k routing ids [T, k]: the (token, slot)
    pairs ordered by expert, and within an expert by token then slot (a stable sort of
    the flattened ids).  Returns (order [T*k] of flat slot indices t*k + j, offsets
    [E+1]: expert e owns rows offsets[e] .. offsets[e+1]-1)."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return order, offsets


def qmoe_ragged_mm(X_f16, offsets, fc, K, N, block, bits=4, w_round=None) -> np.ndarray:
    """Grouped matmul over experts: rows r in [offsets[e], offsets[e+1]) use expert e,

        y[r] = x[r] . dequant(W_e)^T + b_e      (fp64, unrounded; empty experts skipped)

    X fp16 bits [R, K]; fc = {"W" [E][N][nblk][B/2], "scales" [E][N][nblk], "zp" packed
    or None, "bias" fp16 [E][N] or None}.  w_round names the declared rounding of the
    dequantized weights (e.g. "f16" for the matrix-core operand)."""
    X = f16_bits_to_f64(X_f16)
    R = X.shape[0]
    y = np.zeros((R, N))
    offsets = np.asarray(offsets, dtype=np.int64)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        w = _round_operand(_expert_dequant(fc, e, bits, K, block, N).astype(np.float64), w_round)
        y[r0:r1] = X[r0:r1] @ w.T
        if fc.get("bias") is not None:
            y[r0:r1] += f16_bits_to_f64(np.asarray(fc["bias"])[e])[None, :]
    return y


# ---------------------------------------------------------------------------
# Quantize -> dequantize round trip  ([P1] "What", commit 4: fake_quantize
# exactly equal to the unfused Q -> DQ chain)
# ---------------------------------------------------------------------------

def div_f32(x, s) -> np.ndarray:
    """IEEE fp32 division x / s, correctly rounded (numpy's float32 divide)."""
    return np.asarray(x, dtype=np.float32) / np.asarray(s, dtype=np.float32)


def code_dtype(bits: int):
    return np.uint8 if bits <= 8 else np.uint16


def quantize_linear(x_f32, scale_f32, zp, bits):
    """Unfused Q (ONNX QuantizeLinear): q = saturate(round-half-even(fp32(x / s)) + zp)
    into [0, 2^bits - 1] (the addition exact in fp64); a NaN quotient gives code 0.
    Codes are uint8 for bits <= 8, else uint16."""
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        t = div_f32(x_f32, scale_f32).astype(np.float64)
        r = np.rint(t) + float(zp)
    r = np.where(np.isnan(r), 0.0, np.clip(r, 0.0, float((1 << bits) - 1)))
    return r.astype(code_dtype(bits))


def dequantize_linear(q, scale_f32, zp) -> np.ndarray:
    """Unfused DQ (ONNX DequantizeLinear): x = fp32((q - zp) * s); q - zp is exact."""
    d = np.asarray(q, dtype=np.float64) - float(zp)
    return to_f32(d * np.asarray(scale_f32, dtype=np.float32).astype(np.float64))


def pack_codes(q, bits: int, block: int) -> np.ndarray:
    """Pack codes q[N, K] into [N][nblk][block*bits/8], LSB-first bit streams, zero
    padding (bits = 8: signed codes stored as their two's-complement bytes)."""
    if bits == 8:
        q8 = np.asarray(q).astype(np.int64).astype(np.int8).view(np.uint8)
    else:
        q8 = np.asarray(q).astype(np.uint8)
    N, K = q8.shape
    nblk = (K + block - 1) // block
    qp = np.zeros((N, nblk * block), dtype=np.uint16)
    qp[:, :K] = q8
    qp = qp.reshape(N, nblk, block)
    nbytes = block * bits // 8
    out = np.zeros((N, nblk, nbytes + 1), dtype=np.uint16)
    for j in range(block):
        pos = j * bits
        v = qp[..., j] << np.uint16(pos % 8)
        out[..., pos // 8] |= v & np.uint16(0xFF)
        out[..., pos // 8 + 1] |= v >> np.uint16(8)
    return out[..., :nbytes].astype(np.uint8)


def fake_quantize(x_f32, scale_f32, zp, bits):
    """Fused Q -> DQ ([P1] "What", commit 4): x_hat = fp32((c - zp) * s) with
    c = clamp(rint(fp32(x / s)) + zp, 0, 2^bits - 1) (a NaN quotient gives c = 0)."""
    s = np.asarray(scale_f32, dtype=np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        code = np.rint(div_f32(x_f32, scale_f32).astype(np.float64)) + float(zp)
    code = np.where(np.isnan(code), 0.0, np.clip(code, 0.0, float((1 << bits) - 1)))
    return to_f32(to_f32(code - zp).astype(np.float64) * s)


# ---------------------------------------------------------------------------
# Quantized activation ops and the quantized SwiGLU chain  ([P1] "Why": the
# per-layer chain Q(gate) -> qsigmoid -> 2x qmul -> Q(up) -> DQ; "What", commit 4:
# a fused quantized SwiGLU exactly equal to the unfused chain)
# ---------------------------------------------------------------------------

def sigmoid_f32(v_f32) -> np.ndarray:
    """Logistic function of fp32 inputs, computed in fp64 and rounded once to fp32."""
    v = np.asarray(v_f32, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        return to_f32(1.0 / (1.0 + np.exp(-v)))


def qsigmoid(q_in, s_in, z_in, s_out, z_out, bits):
    """Quantized sigmoid: Q(sigmoid(DQ(q_in)); s_out, z_out)."""
    return quantize_linear(sigmoid_f32(dequantize_linear(q_in, s_in, z_in)), s_out, z_out, bits)


def qmul(qa, sa, za, qb, sb, zb, sc, zc, bits):
    """Quantized product: Q(fp32(DQ(qa) * DQ(qb)); sc, zc) (the fp32 product is one rounding)."""
    p = to_f32(dequantize_linear(qa, sa, za).astype(np.float64) * dequantize_linear(qb, sb, zb).astype(np.float64))
    return quantize_linear(p, sc, zc, bits)


def qswiglu(gate_f32, up_f32, qp, bits):
    """Quantized SwiGLU chain, in the order of the activation graph:

        g = Q(gate; gate params)
        t = qsigmoid(g -> sigmoid params)
        m = qmul(g, t -> silu params)          (silu = gate * sigmoid(gate))
        u = Q(up; up params)
        h = qmul(m, u -> out params)
        y = DQ(h; out params)                   (fp32)

    qp: five (scale, zero_point) pairs: gate, sigmoid, silu, up, out."""
    (sg, zg), (st, zt), (sm, zm), (su, zu), (sh, zh) = qp
    g = quantize_linear(gate_f32, sg, zg, bits)
    t = qsigmoid(g, sg, zg, st, zt, bits)
    m = qmul(g, sg, zg, t, st, zt, sm, zm, bits)
    u = quantize_linear(up_f32, su, zu, bits)
    h = qmul(m, sm, zm, u, su, zu, sh, zh, bits)
    return dequantize_linear(h, sh, zh)


# ---------------------------------------------------------------------------
# Error measures used by the gates
# ---------------------------------------------------------------------------

def rel_l2(y, ref) -> float:
    """||y - ref||_2 / ||ref||_2 (absolute L2 when ||ref|| = 0)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.linalg.norm((y - ref).ravel()))
    den = float(np.linalg.norm(ref.ravel()))
    return num / den if den > 0 else num
