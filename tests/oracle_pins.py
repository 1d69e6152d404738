"""Pins of the oracle against things other than itself.

Each pin takes the oracle module `O` as an argument so that the planted-mistake
test can run the same pins against deliberately broken copies of the oracle and
check that at least one pin fails for each plausible mistake.

The pins use: exact rational arithmetic (fractions.Fraction) on tiny inputs with
codes read from a bit string built independently of the oracle's shifts; closed
forms (all-ones and one-hot activations, constant codes); invariants stated on
the pages (fused Q->DQ equals the unfused chain; a linear codebook reproduces the
affine dequant); and library routines (torch's fp32->bf16 cast, math.exp).
"""
from __future__ import annotations

import math
from fractions import Fraction as Fr

import numpy as np

from gemm_qmm_nbits_amd import inputs as gen


# ---------------------------------------------------------------------------
# independent helpers (no oracle code)
# ---------------------------------------------------------------------------

def _signed(v, bits):
    """8-bit fields are two's-complement codes."""
    return v - 256 if bits == 8 and v >= 128 else v


def bitstring_codes(W, bits, K, block):
    """Codes by building each block's bit stream as a string, bit 0 of byte 0 first."""
    W = np.asarray(W)
    N = W.shape[0]
    out = np.zeros((N, K), dtype=np.int64)
    for n in range(N):
        streams = ["".join(format(int(x), "08b")[::-1] for x in W[n, b]) for b in range(W.shape[1])]
        for k in range(K):
            b, j = divmod(k, block)
            field = streams[b][j * bits:(j + 1) * bits]   # least significant bit first
            out[n, k] = _signed(int(field[::-1], 2), bits)
    return out


def bitstring_zp(zp_packed, bits, nblk):
    zp_packed = np.asarray(zp_packed)
    out = np.zeros((zp_packed.shape[0], nblk), dtype=np.int64)
    for n in range(zp_packed.shape[0]):
        s = "".join(format(int(x), "08b")[::-1] for x in zp_packed[n])
        for b in range(nblk):
            out[n, b] = _signed(int(s[b * bits:(b + 1) * bits][::-1], 2), bits)
    return out


def fr16(bits16):
    return Fr(float(np.uint16(bits16).view(np.float16)))


def fr32(x):
    return Fr(float(np.float32(x)))


def exact_zp(p, n, b):
    bits = p["bits"]
    mode = p["zp_mode"]
    if mode in ("packed8", "packed"):
        nblk = gen.nblocks(p["K"], p["block"])
        return Fr(int(bitstring_zp(p["zp"][n:n + 1], bits, nblk)[0, b]))
    if mode in ("f16_uniform", "f16"):
        return fr16(p["zp"][n, b])
    return Fr(0) if bits == 8 else Fr(1 << (bits - 1))   # unsigned codes: the middle code


def zp_args(O, p):
    mode = p["zp_mode"]
    if mode in ("packed8", "packed"):
        return dict(zp=p["zp"], zp_kind=O.ZP_PACKED)
    if mode in ("f16_uniform", "f16"):
        return dict(zp=p["zp"], zp_kind=O.ZP_F16)
    return dict(zp=None, zp_kind=O.ZP_NONE)


def fr_round(x, mant_bits, emin):
    """Nearest binary float with `mant_bits` significant bits and minimum normal
    exponent `emin` (subnormals below it), ties to even, for a Fraction x.
    Written from the definition: pick the spacing of x's binade, round the
    quotient.  fp16: (11, -14); bf16: (8, -126)."""
    if x == 0:
        return Fr(0)
    sign = -1 if x < 0 else 1
    ax = abs(x)
    # exponent e with 2^e <= ax < 2^(e+1)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    if Fr(2) ** e > ax:
        e -= 1
    e = max(e, emin)
    ulp = Fr(2) ** (e - mant_bits + 1)
    q = ax / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fr(1, 2) or (r == Fr(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def row_shift(row_values):
    """Exponent s with 2^14 <= max|a| * 2^s < 2^15, at most 126 (0 for a zero row)."""
    mx = max(abs(v) for v in row_values)
    if mx == 0:
        return 0
    s = 0
    while mx * Fr(2) ** s >= 2 ** 15:
        s -= 1
    while mx * Fr(2) ** s < 2 ** 14:
        s += 1
    return min(s, 126)


def fr_rint(t):
    """Round a Fraction to the nearest integer, ties to even."""
    r = t.numerator // t.denominator
    frac = t - r
    return r + 1 if frac > Fr(1, 2) or (frac == Fr(1, 2) and r % 2 == 1) else r


def ref_quantize(x, s, zp, bits):
    """QuantizeLinear from its definition: the quotient rounded to fp32 (24 significant
    bits), then to an integer (ties to even), plus the zero point, saturated."""
    xf, sf = float(np.float32(x)), float(np.float32(s))
    if math.isnan(xf):
        return 0
    if math.isinf(xf):
        return (1 << bits) - 1 if (xf > 0) == (sf > 0) else 0
    t = fr_round(Fr(xf) / Fr(sf), 24, -126)
    return min(max(fr_rint(t) + zp, 0), (1 << bits) - 1)


def ref_dequantize(q, s, zp):
    return fr_round((Fr(int(q)) - zp) * Fr(float(np.float32(s))), 24, -126)


def ref_sigmoid(v):
    """fp32 rounding of 1 / (1 + e^-v) with e^-v from math.exp."""
    return fr_round(1 / (1 + Fr(math.exp(-float(v)))), 24, -126)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_unpack_exhaustive(O):
    """Every byte value at every field position (bits 2, 4 and signed 8), and every pair of
    neighbouring byte values under each 3-bit field that crosses a byte, vs the bit
    string; pack is the inverse of unpack."""
    for bits in (2, 4, 8):
        block = 16
        blob = block * bits // 8
        W = np.zeros((256, 1, blob), dtype=np.uint8)
        W[:, 0, :] = np.arange(256, dtype=np.uint8)[:, None]
        got = O.unpack_codes(W, bits, block, block)
        want = bitstring_codes(W, bits, block, block)
        assert np.array_equal(got.astype(np.int64), want), f"unpack bits={bits}"
        # pack is the inverse of unpack on full blocks
        assert np.array_equal(O.pack_codes(got, bits, block), W), f"pack bits={bits}"
    # 3-bit codes: 8 codes per 3 bytes, fields 2 and 5 cross a byte boundary
    block = 16
    pairs = np.array([(a, b) for a in range(0, 256, 3) for b in range(0, 256, 5)], dtype=np.uint8)
    W = np.zeros((len(pairs), 1, 6), dtype=np.uint8)
    for off in (0, 1, 3, 4):   # every byte pair of the block (bytes 2 and 5 end groups)
        W[:, 0, off], W[:, 0, off + 1] = pairs[:, 0], pairs[:, 1]
    W[:, 0, 2] ^= pairs[:, 1][::-1]
    W[:, 0, 5] ^= pairs[:, 0][::-1]
    got = O.unpack_codes(W, 3, block, block)
    want = bitstring_codes(W, 3, block, block)
    assert np.array_equal(got.astype(np.int64), want), "unpack bits=3"
    assert np.array_equal(O.pack_codes(got, 3, block), W), "pack bits=3"
    # packed zero points use the same stream
    zp = np.arange(0, 256, 7, dtype=np.uint8).reshape(-1, 1).repeat(3, axis=1) ^ np.array([0, 0x5A, 0xC3], dtype=np.uint8)
    for bits, nblk in ((3, 8), (8, 3), (4, 6), (2, 12)):
        assert np.array_equal(O.unpack_zero_points(zp, bits, nblk).astype(np.int64),
                              bitstring_zp(zp, bits, nblk)), f"zp bits={bits}"


def pin_nbits_bruteforce(O, seed=7):
    """Tiny MatMulNBits problems vs exact rationals (ragged last block, all zp kinds)."""
    worst = 0.0
    cases = [
        (2, 70, 3, 2, 32, "packed"), (2, 130, 3, 2, 64, "f16_uniform"), (3, 96, 2, 4, 64, "packed8"),
        (1, 100, 4, 4, 32, "packed"), (2, 64, 2, 2, 16, "none"), (2, 48, 3, 4, 16, "f16"),
        (2, 100, 3, 3, 32, "packed"), (1, 64, 2, 3, 64, "none"), (2, 70, 2, 3, 32, "f16"),
        (2, 70, 3, 8, 16, "packed"), (1, 64, 2, 8, 32, "none"), (2, 40, 2, 8, 16, "f16"),
    ]
    for ci, (M, K, N, bits, block, zp) in enumerate(cases):
        p = gen.nbits_problem(M, K, N, bits, block, seed=seed + ci, zp=zp, bias=(ci % 2 == 0),
                              scale_range=(0.01, 0.05))
        if zp == "f16":  # keep (q - zp) exact in fp32: zero points on a 1/64 grid
            z = np.round(O.f16_bits_to_f64(p["zp"]) * 64) / 64
            p["zp"] = z.astype(np.float16).view(np.uint16)
        q = bitstring_codes(p["W"], bits, K, block)
        nblk = gen.nblocks(K, block)
        w_exact = [[(Fr(int(q[n, k])) - exact_zp(p, n, k // block)) * fr16(p["scales"][n, k // block])
                    for k in range(K)] for n in range(N)]
        w_or = O.dequant_nbits(p["W"], bits, K, block, p["scales"], **zp_args(O, p))
        for n in range(N):
            for k in range(K):
                assert Fr(float(w_or[n, k])) == w_exact[n][k], ("dequant", ci, n, k)
        y = O.qmm_nbits(p["A"], "f32", p["W"], bits, K, block, p["scales"], bias=p["bias"],
                        **zp_args(O, p))
        for m in range(M):
            for n in range(N):
                acc = sum(fr32(p["A"][m, k]) * w_exact[n][k] for k in range(K))
                if p["bias"] is not None:
                    acc += fr32(p["bias"][n])
                mag = sum(abs(float(fr32(p["A"][m, k]) * w_exact[n][k])) for k in range(K)) + 1e-30
                err = abs(float(Fr(float(y[m, n])) - acc)) / mag
                worst = max(worst, err)
                assert err < 1e-13, ("nbits sum", ci, m, n, err)
        assert nblk >= 1
    return worst


def pin_nbits_closed_forms(O, seed=11):
    """All-ones A -> per-row sums; one-hot A -> a column; constant codes."""
    K, N, block = 200, 5, 64
    nblk = gen.nblocks(K, block)
    for bits in (2, 4):
        p = gen.nbits_problem(1, K, N, bits, block, seed=seed + bits, zp="packed")
        zpc = bitstring_zp(p["zp"], bits, nblk)
        q = bitstring_codes(p["W"], bits, K, block)
        ones = np.ones((1, K), dtype=np.float32)
        y = O.qmm_nbits(ones, "f32", p["W"], bits, K, block, p["scales"], p["zp"], O.ZP_PACKED)
        for n in range(N):
            want = Fr(0)
            for b in range(nblk):
                ks = range(b * block, min(K, (b + 1) * block))
                want += fr16(p["scales"][n, b]) * (sum(int(q[n, k]) for k in ks) - len(ks) * int(zpc[n, b]))
            assert abs(float(Fr(float(y[0, n])) - want)) <= 1e-12 * (1 + abs(float(want))), ("ones", bits, n)
        for k in (0, 1, block - 1, block, K - 1):
            a = np.zeros((1, K), dtype=np.float32)
            a[0, k] = 1.0
            y = O.qmm_nbits(a, "f32", p["W"], bits, K, block, p["scales"], p["zp"], O.ZP_PACKED)
            for n in range(N):
                want = (int(q[n, k]) - int(zpc[n, k // block])) * fr16(p["scales"][n, k // block])
                assert Fr(float(y[0, n])) == want, ("one-hot", bits, k, n)
        # constant code c everywhere: y = (c - zp) * sum_b s_b * sum_{k in b} a_k
        c = (1 << bits) - 1
        byte = 0
        for f in range(8 // bits):
            byte |= c << (f * bits)
        Wc = np.full_like(p["W"], byte)
        a = p["A"]
        y = O.qmm_nbits(a, "f32", Wc, bits, K, block, p["scales"], None, O.ZP_UNIFORM, uniform_zp=1.5)
        for n in range(N):
            want = sum((Fr(c) - Fr(3, 2)) * fr16(p["scales"][n, b]) *
                       sum(fr32(a[0, k]) for k in range(b * block, min(K, (b + 1) * block)))
                       for b in range(nblk))
            assert abs(float(Fr(float(y[0, n])) - want)) <= 1e-12 * (1 + abs(float(want))), ("const", n)


def pin_codebook_bruteforce(O, seed=13):
    """Tiny codebook problems vs exact rationals, bf16 and fp16 activations."""
    for ci, (M, K, N, a_dtype) in enumerate([(2, 128, 3, "bf16"), (1, 96, 4, "f16"), (3, 64, 2, "f32")]):
        p = gen.codebook_problem(M, K, N, seed=seed + ci, a_dtype=a_dtype, bias=(ci == 1))
        q = bitstring_codes(p["W"], 4, K, 64)
        cb = [fr32(v) for v in p["codebook"]]
        w_or = O.dequant_codebook4(p["W"], K, 64, p["absmax"], p["codebook"])
        if a_dtype == "bf16":
            a = [[Fr(float((np.uint32(v) << np.uint32(16)).view(np.float32))) for v in row] for row in p["A"]]
        elif a_dtype == "f16":
            a = [[fr16(v) for v in row] for row in p["A"]]
        else:
            a = [[fr32(v) for v in row] for row in p["A"]]
        for n in range(N):
            for k in range(K):
                exact = cb[int(q[n, k])] * fr32(p["absmax"][n, k // 64])
                # w is the fp32 rounding of the exact product
                assert abs(Fr(float(w_or[n, k])) - exact) <= abs(exact) * Fr(1, 1 << 24), ("cb dq", ci, n, k)
        y = O.qmm_codebook4(p["A"], a_dtype, p["W"], K, 64, p["absmax"], p["codebook"], bias=p["bias"])
        for m in range(M):
            for n in range(N):
                acc = sum(a[m][k] * Fr(float(w_or[n, k])) for k in range(K))
                if p["bias"] is not None:
                    acc += fr16(p["bias"][n])
                mag = sum(abs(float(a[m][k] * Fr(float(w_or[n, k])))) for k in range(K)) + 1e-30
                assert abs(float(Fr(float(y[m, n])) - acc)) / mag < 1e-13, ("cb sum", ci, m, n)


def pin_codebook_linear_equals_affine(O, seed=17):
    """codebook[i] = (i - 8)/8 with absmax = 8*s reproduces 4-bit dequant with zp 8."""
    K, N, block = 192, 6, 64
    p = gen.nbits_problem(2, K, N, 4, block, seed=seed, zp="packed8")
    cb = ((np.arange(16) - 8) / 8.0).astype(np.float32)
    s = O.f16_bits_to_f64(p["scales"])
    absmax = (8.0 * s).astype(np.float32)
    w_aff = O.dequant_nbits(p["W"], 4, K, block, p["scales"], p["zp"], O.ZP_PACKED)
    w_cb = O.dequant_codebook4(p["W"], K, block, absmax, cb)
    assert np.array_equal(w_aff.view(np.uint32), w_cb.view(np.uint32))
    y_aff = O.qmm_nbits(p["A"], "f32", p["W"], 4, K, block, p["scales"], None, O.ZP_NONE)
    y_cb = O.qmm_codebook4(p["A"], "f32", p["W"], K, block, absmax, cb)
    assert np.allclose(y_aff, y_cb, rtol=1e-14, atol=1e-14)


def pin_fake_quant_chain(O, seed=19):
    """Fused Q->DQ equals quantize -> pack -> unpack -> dequant, bit for bit."""
    rng = np.random.default_rng(seed)
    for bits in (2, 4):
        K, N, block = 256, 8, 64
        nblk = K // block
        s16 = rng.uniform(0.005, 0.05, size=(N, nblk)).astype(np.float16)
        s32 = s16.astype(np.float32)
        x = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
        x[0, :8] = [1e3, -1e3, 0.0, -0.0, 1e-9, s32[0, 0] * 0.5, s32[0, 0] * 1.5, -s32[0, 0] * 2.5]
        zp_int = 1 << (bits - 1)
        s_full = np.repeat(s32, block, axis=1)
        fused = O.fake_quantize(x, s_full, zp_int, bits)
        q = O.quantize_linear(x, s_full, zp_int, bits)
        packed = O.pack_codes(q, bits, block)
        chain = O.dequant_nbits(packed, bits, K, block, s16.view(np.uint16), None, O.ZP_NONE)
        assert np.array_equal(fused.view(np.uint32), chain.view(np.uint32)), bits
        # integer zero point: Q is saturate(round-half-even(x / s) + zp) (QuantizeLinear),
        # with x / s the correctly rounded fp32 quotient
        for i in range(64):
            assert int(q[1, i]) == ref_quantize(x[1, i], s_full[1, i], zp_int, bits)


def pin_bf16_rounding(O, seed=23):
    """Oracle fp32 -> bf16 rounding vs torch's cast (random, ties, specials)."""
    import torch

    rng = np.random.default_rng(seed)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, size=5000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    specials = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001,
                         0x007FFFFF, 0x3F808000, 0x3F818000, 0x7F7F8000], dtype=np.uint32)
    allu = np.concatenate([u, ties, specials])
    x = allu.view(np.float32)
    x = x[~np.isnan(x)]
    got = O.f32_to_bf16_bits(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    nan = O.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(O.bf16_bits_to_f64(nan)[0])


def pin_f16_rounding(O, seed=29):
    """fp64 -> fp16 cast: midpoints between neighbours round to the even one."""
    h = np.arange(0, 0x7BFF, dtype=np.uint16)  # positive finite, each with a successor
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2.0
    got = O.to_f16(mid).view(np.uint16)
    want = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    # just past a midpoint: one rounding goes away from the midpoint (a cast that
    # rounds to fp32 first would land on the midpoint and then round to even)
    above = mid + (hi - lo) * 2.0 ** -30
    below = mid - (hi - lo) * 2.0 ** -30
    assert np.array_equal(O.to_f16(above).view(np.uint16), (h + 1).astype(np.uint16))
    assert np.array_equal(O.to_f16(below).view(np.uint16), h)
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(10000) * 100
    r = O.to_f16(v).astype(np.float64)
    # the nearest fp16: no other fp16 is closer
    bits = O.to_f16(v).view(np.uint16).astype(np.int64)
    for d in (-1, 1):
        nb = (bits + d).astype(np.uint16).view(np.float16).astype(np.float64)
        assert np.all(np.abs(v - r) <= np.abs(v - nb))


def pin_swiglu(O):
    """SwiGLU vs math.exp; g = 0 or u = 0 gives 0; silu(-x) = silu(x) - x."""
    g = np.array([-30.0, -3.5, -1.0, -1e-3, 0.0, 1e-3, 0.7, 2.0, 12.0])
    u = np.array([0.5, -2.0, 1.0, 3.0, 5.0, -1.0, 0.25, 0.0, 1.5])
    h = O.swiglu(np.concatenate([g, u]), len(g))
    for i in range(len(g)):
        want = g[i] / (1.0 + math.exp(-g[i])) * u[i]
        assert abs(h[i] - want) <= 1e-15 * (1 + abs(want)), i
    assert h[4] == 0.0 and h[7] == 0.0
    x = np.linspace(-8, 8, 101)
    ones = np.ones_like(x)
    s_pos = O.swiglu(np.concatenate([x, ones]), len(x))
    s_neg = O.swiglu(np.concatenate([-x, ones]), len(x))
    assert np.allclose(s_neg, s_pos - x, rtol=0, atol=1e-14)


def pin_int8_quantizer(O, seed=31):
    """Properties that fix the symmetric per-32 int8 quantizer."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((4, 256)).astype(np.float16).astype(np.float64)
    v[1, 32:64] = 0.0
    q, s = O.quantize_int8_groups(v)
    assert q.dtype == np.int8 and s.shape == (4, 8)
    assert np.all(np.abs(q.astype(np.int64)) <= 127)
    assert np.all(q[1, 32:64] == 0) and s[1, 1] == 0.0
    g = v.reshape(4, 8, 32)
    qg = q.reshape(4, 8, 32).astype(np.int64)
    for r in range(4):
        for b in range(8):
            amax = np.abs(g[r, b]).max()
            if amax == 0:
                continue
            i = int(np.argmax(np.abs(g[r, b])))
            assert abs(qg[r, b, i]) == 127
            assert float(s[r, b]) == float(np.float32(amax / 127.0))
            err = np.abs(g[r, b] - qg[r, b] * float(s[r, b]))
            assert np.all(err <= 0.5 * float(s[r, b]) * (1 + 1e-6) + 1e-12)
    qn, sn = O.quantize_int8_groups(-v)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # monotone in v within a group
    srt = np.sort(v[0, :32])
    qs, _ = O.quantize_int8_groups(srt[None, :])
    assert np.all(np.diff(qs[0].astype(np.int64)) >= 0)


def pin_uniform_zp(O):
    z = np.full((7, 5), np.float16(1.5)).view(np.uint16)
    assert O.fp16_uniform_value(z) == (True, 1.5)
    z2 = z.copy()
    z2[6, 4] = np.float16(1.5 + 2**-9).view(np.uint16)
    assert O.fp16_uniform_value(z2)[0] is False
    zero = np.zeros((3, 3), dtype=np.uint16)
    negz = zero.copy()
    negz[1, 1] = 0x8000
    assert O.fp16_uniform_value(zero) == (True, 0.0)
    assert O.fp16_uniform_value(negz)[0] is False
    assert O.fp16_uniform_value(np.full((2, 2), 0x7E00, dtype=np.uint16))[0] is False
    assert O.fp16_uniform_value(np.zeros((0,), dtype=np.uint16))[0] is False


def _qmoe_exact(O, p, mode):
    """Per-slot brute force of the MoE decode with rationals; sigmoid via math.exp."""
    H, I, E, k, block = p["H"], p["I"], p["E"], p["k"], p["block"]
    T = p["T"]
    out = np.zeros((T, H))

    def dq(fc, e, n_out, k_in):
        q = bitstring_codes(fc["W"][e], 4, k_in, block)
        nblk = gen.nblocks(k_in, block)
        z = bitstring_zp(fc["zp"][e], 4, nblk) if fc["zp"] is not None else np.full((n_out, nblk), 8)
        return [[(Fr(int(q[n, kk])) - int(z[n, kk // block])) * fr16(fc["scales"][e, n, kk // block])
                 for kk in range(k_in)] for n in range(n_out)]

    for t in range(T):
        x = [fr16(v) for v in p["X"][t]]
        if mode == "int8":
            xq, xs = O.quantize_int8_groups(O.f16_bits_to_f64(p["X"][t]))
            x = [Fr(int(xq[i])) * fr32(xs[i // 32]) for i in range(H)]
        acc = [Fr(0)] * H
        for j in range(k):
            e = int(p["ids"][t, j])
            w1 = dq(p["fc1"], e, 2 * I, H)
            w2 = dq(p["fc2"], e, H, I)
            gu = [sum(w1[n][i] * x[i] for i in range(H)) for n in range(2 * I)]
            if p["fc1"]["bias"] is not None:
                gu = [gu[n] + fr16(p["fc1"]["bias"][e, n]) for n in range(2 * I)]
            h = []
            for i in range(I):
                gf = float(gu[i])
                hv = gf / (1.0 + math.exp(-gf)) * float(gu[I + i])
                h.append(Fr(float(np.float16(hv))))
            if mode == "int8":
                hq, hs = O.quantize_int8_groups(np.array([float(v) for v in h]))
                h = [Fr(int(hq[i])) * fr32(hs[i // 32]) for i in range(I)]
            r = fr32(p["rw"][t, j])
            for n in range(H):
                z = sum(w2[n][i] * h[i] for i in range(I))
                if p["fc2"]["bias"] is not None:
                    z += fr16(p["fc2"]["bias"][e, n])
                acc[n] += r * z
        out[t] = [float(v) for v in acc]
    return out


def pin_qmoe_bruteforce(O, seed=37):
    """Tiny MoE decode vs rationals (fp and int8 modes, zp and bias on/off, T = 2)."""
    for ci, (zp, bias, mode, block) in enumerate([(True, True, "fp", 32), (False, False, "fp", 64),
                                                  (True, False, "int8", 32), (False, True, "int8", 64)]):
        p = gen.qmoe_problem(2, 64, 32, 3, 2, block, seed=seed + ci, zp=zp, bias=bias,
                             scale_range=(0.05, 0.2))
        want = _qmoe_exact(O, p, mode)
        got = O.qmoe_decode(p["X"], p["ids"], p["rw"], p["fc1"], p["fc2"], 64, 32, block, mode=mode)
        assert np.allclose(got, want, rtol=1e-9, atol=1e-9), (ci, np.abs(got - want).max())


def pin_qmoe_composition(O, seed=41):
    """k = 1, weight 1: the MoE decode is fc2(fp16(SwiGLU(fc1(x)))) through qmm_nbits;
    weight 0 gives 0; all codes equal to the zero point give sum_j r_j * b2."""
    H, I, E, block = 128, 64, 4, 32
    p = gen.qmoe_problem(1, H, I, E, 1, block, seed=seed, zp=True, bias=True)
    e = int(p["ids"][0, 0])
    one = np.ones((1, 1), dtype=np.float32)
    got = O.qmoe_decode(p["X"], p["ids"], one, p["fc1"], p["fc2"], H, I, block)
    gu = O.qmm_nbits(p["X"], "f16", p["fc1"]["W"][e], 4, H, block, p["fc1"]["scales"][e],
                     p["fc1"]["zp"][e], O.ZP_PACKED, bias=p["fc1"]["bias"][e], bias_dtype="f16")
    g, u = gu[0, :I], gu[0, I:]
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float16).view(np.uint16)[None, :]
    want = O.qmm_nbits(h, "f16", p["fc2"]["W"][e], 4, I, block, p["fc2"]["scales"][e],
                       p["fc2"]["zp"][e], O.ZP_PACKED, bias=p["fc2"]["bias"][e], bias_dtype="f16")
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    zero = np.zeros((1, 1), dtype=np.float32)
    assert np.all(O.qmoe_decode(p["X"], p["ids"], zero, p["fc1"], p["fc2"], H, I, block) == 0.0)
    # every code equal to its zero point: only the fc2 bias survives
    p2 = gen.qmoe_problem(1, H, I, E, 3, block, seed=seed + 1, zp=True, bias=True)
    for fc in ("fc1", "fc2"):
        p2[fc]["W"][:] = 0x55
        p2[fc]["zp"][:] = 0x55
    got = O.qmoe_decode(p2["X"], p2["ids"], p2["rw"], p2["fc1"], p2["fc2"], H, I, block)
    want = sum(float(np.float32(p2["rw"][0, j])) *
               O.f16_bits_to_f64(p2["fc2"]["bias"][int(p2["ids"][0, j])]) for j in range(3))
    assert np.allclose(got[0], want, rtol=1e-14, atol=0)


def pin_round_operand(O, seed=43):
    """Declared operand roundings of the matrix-core paths vs exact rationals.

    A' is the per-row pre-scaled fp16 rounding (f16_rows), W' the fp16 rounding of
    the exact dequantized weight; each is checked alone and together, on rows whose
    largest value overflows fp16, rows of tiny values and ordinary rows.  Integer
    activations up to 2^11 make the activation rounding the identity."""
    rng = np.random.default_rng(seed)
    K, N, block = 40, 3, 16
    p = gen.nbits_problem(4, K, N, 4, block, seed=seed, zp="packed", scale_range=(0.01, 0.05))
    A = rng.standard_normal((4, K))
    A[1] *= 3e5            # largest values past the fp16 range
    A[2] *= 1e-7           # every value below the smallest normal fp16
    A[3, 5] = 7e4          # one large value in a row of ordinary ones
    A = A.astype(np.float32)
    w = O.dequant_nbits(p["W"], 4, K, block, p["scales"], p["zp"], O.ZP_PACKED)
    a_fr = [[fr32(A[m, k]) for k in range(K)] for m in range(4)]
    w_fr = [[Fr(float(w[n, k])) for k in range(K)] for n in range(N)]
    a16 = []
    for m in range(4):
        s = row_shift(a_fr[m])
        assert s == int(O.row_prescale_exponents(A.astype(np.float64))[m]), ("shift", m)
        a16.append([fr_round(v * Fr(2) ** s, 11, -14) / Fr(2) ** s for v in a_fr[m]])
    w16 = [[fr_round(v, 11, -14) for v in row] for row in w_fr]
    for a_round, w_round, aa, ww in ((None, None, a_fr, w_fr), ("f16_rows", None, a16, w_fr),
                                     (None, "f16", a_fr, w16), ("f16_rows", "f16", a16, w16)):
        y = O.qmm_nbits(A, "f32", p["W"], 4, K, block, p["scales"], p["zp"], O.ZP_PACKED,
                        a_round=a_round, w_round=w_round)
        for m in range(4):
            for n in range(N):
                exact = sum(aa[m][k] * ww[n][k] for k in range(K))
                mag = sum(abs(float(aa[m][k] * ww[n][k])) for k in range(K)) + 1e-300
                err = abs(float(Fr(float(y[m, n])) - exact)) / mag
                assert err < 1e-13, (a_round, w_round, m, n, err)
    # the pre-scaled rounding keeps every row finite and the tiny row's bits
    r = O._round_operand(A.astype(np.float64), "f16_rows")
    assert np.all(np.isfinite(r))
    assert np.max(np.abs(r[2] / A[2].astype(np.float64) - 1)) < 2.0 ** -11
    # integer activations |a| <= 2^11: the rounding is the identity
    Ai = rng.integers(-2048, 2049, size=(3, K)).astype(np.float64)
    assert np.array_equal(O._round_operand(Ai, "f16_rows"), Ai)
    # bf16 of fp32 values vs the rational rounding to 8 significant bits
    v = (rng.standard_normal(200) * 10.0 ** rng.integers(-3, 4, size=200)).astype(np.float32)
    got = O._round_operand(v.astype(np.float64), "bf16")
    for i in range(len(v)):
        assert Fr(float(got[i])) == fr_round(fr32(v[i]), 8, -126), i
    # the codebook entry applies the same roundings
    pc = gen.codebook_problem(2, K, N, seed=seed + 1, a_dtype="f32", block=block)
    pc["A"] = A[:2].copy()
    wc = O.dequant_codebook4(pc["W"], K, block, pc["absmax"], pc["codebook"])
    yc = O.qmm_codebook4(pc["A"], "f32", pc["W"], K, block, pc["absmax"], pc["codebook"],
                         a_round="f16_rows", w_round="f16")
    for m in range(2):
        for n in range(N):
            exact = sum(a16[m][k] * fr_round(Fr(float(wc[n, k])), 11, -14) for k in range(K))
            mag = sum(abs(float(a16[m][k] * Fr(float(wc[n, k])))) for k in range(K)) + 1e-300
            assert abs(float(Fr(float(yc[m, n])) - exact)) / mag < 1e-13, (m, n)


def pin_rel_l2(O):
    """Relative L2 on closed-form vectors."""
    ref = np.array([3.0, 4.0])
    assert O.rel_l2(ref, ref) == 0.0
    assert O.rel_l2(np.array([3.0, 4.5]), ref) == 0.1                 # 0.5 / 5
    assert O.rel_l2(np.array([0.0, 0.0]), ref) == 1.0
    assert O.rel_l2(np.array([6.0, 8.0]), ref) == 1.0
    m = np.array([[1.0, 2.0], [2.0, 4.0]])                             # norm 5
    assert O.rel_l2(m + np.array([[0.0, 0.0], [0.0, 1.0]]), m) == 0.2  # whole array, not per row
    assert O.rel_l2(np.array([3.0, 4.0]), np.zeros(2)) == 5.0          # absolute when ref = 0
    v = np.array([1.0, -2.0, 2.0])                                     # norm 3
    assert abs(O.rel_l2(v + np.array([0.3, 0.0, 0.0]), v) - 0.1) < 1e-15
    assert abs(O.rel_l2(1e3 * (v + 0.1), 1e3 * v) - O.rel_l2(v + 0.1, v)) < 1e-15


def pin_quantized_ops(O, seed=47):
    """QuantizeLinear / DequantizeLinear, the quantized sigmoid and product, and the
    quantized SwiGLU chain against their definitions in exact rational arithmetic (fp32
    quotients and products rounded from the exact value, ties to even), on random values,
    exact ties, saturation, NaN and infinities; plus closed forms (a zero gate gives 0)."""
    rng = np.random.default_rng(seed)
    for bits in (8, 16):
        qmax = (1 << bits) - 1
        s = np.float32(2.0 ** -6 if bits == 8 else 2.0 ** -12)
        zp = 1 << (bits - 1)
        x = (rng.standard_normal(300) * 1.5).astype(np.float32)
        ties = ((rng.integers(-100, 100, size=40) + 0.5) * float(s)).astype(np.float32)
        specials = np.array([0.0, -0.0, 1e30, -1e30, np.inf, -np.inf, np.nan, float(s) * (qmax + 5)],
                            dtype=np.float32)
        xs = np.concatenate([x, ties, specials])
        q = O.quantize_linear(xs, s, zp, bits)
        assert q.dtype == (np.uint8 if bits == 8 else np.uint16)
        for i, v in enumerate(xs):
            assert int(q[i]) == ref_quantize(v, s, zp, bits), ("Q", bits, i, v)
        # a scale that is not a power of two: the fp32 quotient decides, most visibly for
        # values next to a rounding tie ((k + 1/2) * s rounded to fp32)
        s2 = np.float32(0.0123)
        near = ((rng.integers(-60, 60, size=200) + 0.5) * np.float64(s2)).astype(np.float32)
        # and their fp32 neighbours, a few ulps either side of the tie
        nb = near.view(np.int32)[:, None] + np.arange(-3, 4, dtype=np.int32)[None, :]
        xn = np.concatenate([x, nb.ravel().view(np.float32)])
        q2 = O.quantize_linear(xn, s2, 3, bits)
        for i, v in enumerate(xn):
            assert int(q2[i]) == ref_quantize(v, s2, 3, bits), ("Q s2", bits, i)
        codes = rng.integers(0, qmax + 1, size=200)
        d = O.dequantize_linear(codes, s2, 77)
        for i, c in enumerate(codes):
            assert Fr(float(d[i])) == ref_dequantize(c, s2, 77), ("DQ", bits, i)
        # fused Q -> DQ is the chain
        fq = O.fake_quantize(xs, s2, 5, bits)
        ch = O.dequantize_linear(O.quantize_linear(xs, s2, 5, bits), s2, 5)
        assert np.array_equal(fq.view(np.uint32), ch.view(np.uint32))
        # quantized sigmoid and product, one code at a time
        sin, zin = np.float32(8.0 / qmax), zp
        sout, zout = np.float32(1.0 / qmax), 0
        qi = rng.integers(0, qmax + 1, size=200)
        qs = O.qsigmoid(qi, sin, zin, sout, zout, bits)
        for i, c in enumerate(qi):
            t = fr_round(Fr(float(ref_dequantize(c, sin, zin))), 24, -126)
            y = ref_sigmoid(float(t))
            assert int(qs[i]) == min(max(fr_rint(fr_round(y / Fr(float(sout)), 24, -126)) + zout, 0), qmax), i
        assert np.all(np.diff(O.qsigmoid(np.arange(qmax + 1), sin, zin, sout, zout, bits).astype(np.int64)) >= 0)
        qa = rng.integers(0, qmax + 1, size=200)
        qb = rng.integers(0, qmax + 1, size=200)
        sa, sb, sc = np.float32(0.031), np.float32(0.017), np.float32(0.0093)
        qc = O.qmul(qa, sa, 100, qb, sb, 9, sc, 40, bits)
        for i in range(200):
            prod = fr_round(ref_dequantize(qa[i], sa, 100) * ref_dequantize(qb[i], sb, 9), 24, -126)
            assert int(qc[i]) == min(max(fr_rint(fr_round(prod / Fr(float(sc)), 24, -126)) + 40, 0), qmax), i
        # the SwiGLU chain, element by element
        qp = [(np.float32(6.0 / qmax), zp), (np.float32(1.0 / qmax), 0), (np.float32(7.0 / qmax), zp),
              (np.float32(6.0 / qmax), zp), (np.float32(9.0 / qmax), zp)]
        gate = (rng.standard_normal(150) * 1.2).astype(np.float32)
        up = (rng.standard_normal(150) * 1.2).astype(np.float32)
        gate[:3] = [0.0, 100.0, -100.0]
        y = O.qswiglu(gate, up, qp, bits)
        for i in range(150):
            g = ref_quantize(gate[i], qp[0][0], qp[0][1], bits)
            gd = ref_dequantize(g, *qp[0])
            t = min(max(fr_rint(fr_round(ref_sigmoid(float(gd)) / Fr(float(qp[1][0])), 24, -126)) + qp[1][1], 0), qmax)
            m_ = fr_round(gd * ref_dequantize(t, *qp[1]), 24, -126)
            m = min(max(fr_rint(fr_round(m_ / Fr(float(qp[2][0])), 24, -126)) + qp[2][1], 0), qmax)
            u = ref_quantize(up[i], qp[3][0], qp[3][1], bits)
            h_ = fr_round(ref_dequantize(m, *qp[2]) * ref_dequantize(u, *qp[3]), 24, -126)
            h = min(max(fr_rint(fr_round(h_ / Fr(float(qp[4][0])), 24, -126)) + qp[4][1], 0), qmax)
            assert Fr(float(y[i])) == ref_dequantize(h, *qp[4]), ("swiglu", bits, i)
        assert y[0] == 0.0   # a zero gate gives silu 0 and an output of 0


def pin_ragged_mm(O, seed=53):
    """Ragged expert matmul vs exact rationals (ragged last block, zero points, bias, an
    empty expert, a one-row expert); the grouping is a stable sort by expert."""
    rng = np.random.default_rng(seed)
    E, K, N, block = 4, 40, 3, 32
    ids = np.array([[2, 0], [2, 3], [0, 2], [3, 2]], dtype=np.int32)   # expert 1 unused
    order, offsets = O.group_by_expert(ids, E)
    assert list(offsets) == [0, 2, 2, 6, 8]
    assert list(order) == [1, 4, 0, 2, 5, 7, 3, 6]
    p = gen.qmoe_problem(1, K, N // 2, E, 1, block, seed=seed, zp=True, bias=True)
    fc = p["fc1"]   # [E][N][...] with N = 2 * (N // 2) rows ... use the first N rows
    Nn = fc["W"].shape[1]
    X = gen.activations(rng, (8, K), "f16")
    y = O.qmoe_ragged_mm(X, offsets, fc, K, Nn, block)
    nblk = gen.nblocks(K, block)
    for e in range(E):
        q = bitstring_codes(fc["W"][e], 4, K, block)
        z = bitstring_zp(fc["zp"][e], 4, nblk)
        for r in range(int(offsets[e]), int(offsets[e + 1])):
            for n in range(Nn):
                acc = sum(fr16(X[r, k]) * (Fr(int(q[n, k])) - int(z[n, k // block])) *
                          fr16(fc["scales"][e, n, k // block]) for k in range(K))
                acc += fr16(fc["bias"][e, n])
                assert abs(float(Fr(float(y[r, n])) - acc)) <= 1e-12 * (1 + abs(float(acc))), (e, r, n)
    # every row of one expert: the plain MatMulNBits of that expert
    one = np.array([0, 0, 8, 8, 8], dtype=np.int64)
    y1 = O.qmoe_ragged_mm(X, one, fc, K, Nn, block)
    want = O.qmm_nbits(X, "f16", fc["W"][1], 4, K, block, fc["scales"][1], fc["zp"][1], O.ZP_PACKED,
                       bias=fc["bias"][1], bias_dtype="f16")
    assert np.allclose(y1, want, rtol=1e-13, atol=1e-13)


def pin_nested_absmax(O, seed=59):
    """Double-quantized absmax vs exact rationals; a table and scales that make every
    step exact give the plain values; with the offset 0 and scale 1 the table itself."""
    rng = np.random.default_rng(seed)
    na = gen.nested_absmax_inputs(rng, 5, 70, group=64)
    got = O.nested_absmax(na["codes"], na["table"], na["scales"], na["offset"], 64)
    flat = na["codes"].ravel()
    for i in range(flat.size):
        prod = fr_round(fr32(na["table"][flat[i]]) * fr32(na["scales"][i // 64]), 24, -126)
        want = fr_round(prod + fr32(na["offset"]), 24, -126)
        assert Fr(float(got.ravel()[i])) == want, i
    ident = O.nested_absmax(np.arange(256, dtype=np.uint8).reshape(4, 64), na["table"],
                            np.ones(4, dtype=np.float32), 0.0, 64)
    assert np.array_equal(ident.ravel().view(np.uint32), na["table"].view(np.uint32))
    # the codebook matmul on decoded absmax equals the one on the same fp32 values
    p = gen.codebook_problem(2, 200, 5, seed=seed, a_dtype="f32", block=64)
    nb = gen.nested_absmax_inputs(rng, 5, 4, group=8)
    am = O.nested_absmax(nb["codes"], nb["table"], nb["scales"], nb["offset"], 8)
    y = O.qmm_codebook4(p["A"], "f32", p["W"], 200, 64, am, p["codebook"])
    q = bitstring_codes(p["W"], 4, 200, 64)
    for m in range(2):
        for n in range(5):
            acc = sum(fr32(p["A"][m, k]) * fr_round(fr32(p["codebook"][q[n, k]]) * fr32(am[n, k // 64]), 24, -126)
                      for k in range(200))
            assert abs(float(Fr(float(y[m, n])) - acc)) < 1e-12, (m, n)


ALL_PINS = [pin_unpack_exhaustive, pin_nbits_bruteforce, pin_nbits_closed_forms,
            pin_codebook_bruteforce, pin_codebook_linear_equals_affine, pin_fake_quant_chain,
            pin_bf16_rounding, pin_f16_rounding, pin_swiglu, pin_int8_quantizer, pin_uniform_zp,
            pin_qmoe_bruteforce, pin_qmoe_composition, pin_round_operand, pin_rel_l2, pin_quantized_ops,
            pin_ragged_mm, pin_nested_absmax]
