"""GPU parity of qmm_nbits / qmm_dequantize_nbits / qmm_fp16_uniform_value against the oracle."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import inputs as gen
from gemm_qmm_nbits_amd import qmm as Q
from oracle import qmm_oracle as O

from gpu_util import (TOL, NbitsDev, assert_elementwise, dev, dev_act, gamma, host_bits, host_f64, nbits_reference,
                      oracle_zp_kind, say, torch)

pytestmark = pytest.mark.gpu


# --- dequantization: bit-exact ------------------------------------------------

@pytest.mark.parametrize("bits,block,K,zp", [
    (2, 64, 5120, "f16_uniform"), (2, 16, 70, "packed"), (2, 32, 200, "f16"),
    (4, 64, 256, "packed8"), (4, 32, 2880, "packed"), (4, 128, 2880, "none"), (4, 256, 600, "f16"),
])
@pytest.mark.parametrize("out", ["f32", "f16"])
def test_dequant_bit_exact(bits, block, K, zp, out):
    say(f"dequant bits={bits} block={block} K={K} zp={zp} out={out}")
    p = gen.nbits_problem(1, K, 96, bits, block, seed=100 + K + bits, zp=zp)
    d = NbitsDev(p)
    t = torch()
    got = Q.qmm_dequantize_nbits(d.W, d.scales, K, bits, block, d.zp, gpu_kind(zp),
                                 out_dtype=t.float32 if out == "f32" else t.float16)
    t.cuda.synchronize()
    w = O.dequant_nbits(p["W"], bits, K, block, p["scales"], p["zp"], oracle_zp_kind(O, zp))
    if out == "f32":
        assert np.array_equal(host_bits(got).view(np.uint32), w.view(np.uint32))
    else:
        assert np.array_equal(host_bits(got).view(np.uint16), O.to_f16(w).view(np.uint16))


def gpu_kind(zp):
    return {"packed8": Q.QMM_ZP_PACKED, "packed": Q.QMM_ZP_PACKED, "f16_uniform": Q.QMM_ZP_F16,
            "f16": Q.QMM_ZP_F16, "none": Q.QMM_ZP_NONE}[zp]


def test_dequant_exhaustive_scales():
    """Every code x every finite positive fp16 scale x zero points {8, 1.5, 0..15}."""
    t = torch()
    scales = np.arange(1, 0x7C00, dtype=np.uint16)  # all finite positive fp16 patterns
    for bits in (2, 4):
        ncodes = 1 << bits
        block = 16
        # one row per scale; every row holds every code (repeated to fill the block)
        codes = np.tile(np.arange(ncodes, dtype=np.uint8), block // ncodes)[None, :].repeat(len(scales), 0)
        W = O.pack_codes(codes, bits, block)
        for zpv in ([8.0, 1.5] + [float(z) for z in range(16)]) if bits == 4 else [1.5, 2.0, 0.0, 3.0]:
            sc = scales[:, None]
            got = Q.qmm_dequantize_nbits(dev(W), dev(np.ascontiguousarray(sc)), block, bits, block,
                                         None, Q.QMM_ZP_UNIFORM, zpv)
            w = O.dequant_nbits(W, bits, block, block, sc, None, O.ZP_UNIFORM, zpv)
            assert np.array_equal(host_bits(got).view(np.uint32), w.view(np.uint32)), (bits, zpv)
        t.cuda.synchronize()


def test_dequant_matches_fake_quant():
    """GPU dequant of codes packed from the oracle's quantizer == oracle fused Q->DQ."""
    rng = np.random.default_rng(5)
    for bits in (2, 4):
        K, N, block = 512, 64, 64
        s16 = rng.uniform(0.005, 0.05, size=(N, K // block)).astype(np.float16)
        x = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
        s_full = np.repeat(s16.astype(np.float32), block, axis=1)
        zp = 1 << (bits - 1)
        q = O.quantize_linear(x, s_full, zp, bits)
        W = O.pack_codes(q, bits, block)
        got = Q.qmm_dequantize_nbits(dev(W), dev(s16.view(np.uint16)), K, bits, block, None,
                                     Q.QMM_ZP_NONE)
        want = O.fake_quantize(x, s_full, zp, bits)
        assert np.array_equal(host_bits(got).view(np.uint32), want.view(np.uint32))


# --- GEMV path (M <= 8) -------------------------------------------------------

def _bias_args(d):
    """Bias as the oracle takes it: fp32 values, or the stored 16-bit patterns."""
    bias = d.p["bias"]
    if bias is not None and d.c_dtype != "f32":
        return host_bits(d.bias).view(np.uint16), d.c_dtype
    return bias, "f32"


def _check(d, got, label=""):
    """GEMV path: every output column against the exact oracle (relative L2 gate) and
    every element within the bound of the GEMV's arithmetic: fp32 roundings over the
    products and the zero-point fold, plus the 23-bit block fixed point of A."""
    bias, bdt = _bias_args(d)
    r = nbits_reference(O, d.p, bias=bias, bias_dtype=bdt)
    y = host_f64(got)
    err = O.rel_l2(y, r["exact"])
    say(f"  {label} relL2={err:.3e} (tol {TOL[d.c_dtype]:.0e})")
    assert err <= TOL[d.c_dtype], (label, err)
    a = O.activations_f64(d.p["A"], d.p["a_dtype"])
    K = d.p["K"]
    bound = gamma(2 * K + 8) * (r["absdot"] + r["zsdot"]) + 2.0 ** -22 * np.abs(a).max(axis=1)[:, None] * r["wsum"][None, :]
    assert_elementwise(y, r["exact"], bound, d.c_dtype, label)
    return err


def test_tiny_u4_config():
    """Tiny u4 GEMV: M=1, K=256, N=128, block 64, zp code 8, fp32 in/out."""
    p = gen.nbits_problem(1, 256, 128, 4, 64, seed=gen.config_seed(0), zp="packed8")
    d = NbitsDev(p)
    _check(d, d.run(), label="tiny")


@pytest.mark.parametrize("name", list(gen.PHI4_SHAPES))
def test_phi4_u2_decode_full_size(name):
    """phi4-14B 2-bit shapes at M = 1, fp32 A/C, uniform zp 1.5 (full size; sampled oracle rows)."""
    K, N = gen.PHI4_SHAPES[name]
    say(f"phi4 {name} K={K} N={N}")
    p = gen.nbits_problem(1, K, N, 2, 64, seed=gen.config_seed(1, list(gen.PHI4_SHAPES).index(name)),
                          zp="f16_uniform", uniform_zp=1.5, scale_range=(0.01, 0.05))
    d = NbitsDev(p)
    got_u = d.run(uniform=True)
    got_t = d.run(uniform=False)
    torch().cuda.synchronize()
    # the uniform-scalar path and the fp16-tensor path give the same bits
    assert np.array_equal(host_bits(got_u), host_bits(got_t))
    _check(d, got_u, label=name)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 11])
@pytest.mark.parametrize("bits,block,K,N,zp,a,c", [
    (2, 64, 1000, 300, "packed", "f32", "f32"),
    (4, 32, 2880, 257, "packed", "f16", "f16"),
    (4, 128, 2880, 190, "none", "bf16", "bf16"),
    (2, 16, 512, 130, "f16", "f32", "f16"),
    (2, 16, 70, 33, "packed", "f32", "f32"),     # 20-byte rows: generic kernel
    (4, 256, 1536, 64, "f16", "bf16", "f32"),
    (2, 64, 5120, 300, "f16_uniform", "f16", "f16"),   # u2 planes from fp16 activations
    (2, 64, 1000, 260, "packed", "bf16", "f32"),       # u2 planes from bf16 activations
    (2, 32, 2048, 129, "none", "f16", "f32"),
])
def test_gemv_small_shapes(M, bits, block, K, N, zp, a, c):
    say(f"gemv M={M} bits={bits} block={block} K={K} N={N} zp={zp} a={a} c={c}")
    p = gen.nbits_problem(M, K, N, bits, block, seed=7 * M + K, zp=zp, a_dtype=a, bias=(M % 2 == 1))
    d = NbitsDev(p, c_dtype=c)
    if M > 8:  # prefill path: operands rounded to fp16 by declaration
        _check_prefill(d, d.run(), label=f"M={M}")
    else:
        _check(d, d.run(), label=f"M={M}")


def test_repeat_calls_bit_identical():
    """129 calls on the same inputs give the bits of the first call."""
    p = gen.nbits_problem(1, 5120, 7680, 2, 64, seed=77, zp="f16_uniform", scale_range=(0.01, 0.05))
    d = NbitsDev(p)
    first = host_bits(d.run(uniform=True)).copy()
    out = torch().empty_like(d.run(uniform=True))
    for i in range(128):
        d.run(uniform=True, out=out)
        assert np.array_equal(host_bits(out), first), i


def test_every_tiling_candidate_same_bits():
    t = torch()
    p = gen.nbits_problem(3, 4096, 1000, 4, 64, seed=78, zp="packed")
    d = NbitsDev(p)
    outs = []
    try:
        for c in range(Q.num_candidates(Q.ENTRY_NBITS)):
            Q.set_tuning(2, c)
            outs.append(host_bits(d.run()).copy())
            assert Q.tuned_choice(Q.ENTRY_NBITS) == c
    finally:
        Q.set_tuning(0, 0)
    t.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_uniform_zero_point_detection():
    t = torch()
    z = np.full((5120, 80), np.float16(1.5)).view(np.uint16)
    assert Q.qmm_fp16_uniform_value(dev(z)) == (True, 1.5)
    z2 = z.copy()
    z2[4000, 79] = np.float16(1.25).view(np.uint16)
    assert Q.qmm_fp16_uniform_value(dev(z2))[0] is False
    z3 = np.zeros(1000, dtype=np.uint16)
    z3[999] = 0x8000  # -0.0 differs from +0.0 bitwise
    assert Q.qmm_fp16_uniform_value(dev(z3))[0] is False
    assert Q.qmm_fp16_uniform_value(dev(np.full(77, 0x7E00, dtype=np.uint16)))[0] is False
    big = np.full(100352 * 80, np.float16(1.5)).view(np.uint16)
    assert Q.qmm_fp16_uniform_value(dev(big)) == (True, 1.5)
    for arr in (z, z2, z3):
        assert Q.qmm_fp16_uniform_value(dev(arr))[0] == O.fp16_uniform_value(arr)[0]
    t.cuda.synchronize()


def test_pending_error_does_not_fail_call():
    """A HIP error left pending by unrelated earlier work is cleared on entry."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime already loaded by torch
    hip.hipGetLastError.restype = ctypes.c_int
    # hipSetDevice on an invalid ordinal records hipErrorInvalidDevice without touching the GPU
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    assert hip.hipSetDevice(9999) != 0
    p = gen.nbits_problem(1, 512, 64, 4, 64, seed=3, zp="packed8")
    d = NbitsDev(p)
    got = d.run()
    assert O.rel_l2(host_f64(got), d.oracle(O)) <= TOL["f32"]


def test_refused_arguments_on_device():
    t = torch()
    p = gen.nbits_problem(1, 256, 16, 4, 64, seed=4, zp="packed8")
    d = NbitsDev(p)
    with pytest.raises(Q.QmmError) as e:
        Q.qmm_nbits(d.A, d.W, d.scales, 256, 5, 64, d.zp, Q.QMM_ZP_PACKED)
    assert e.value.status == -3
    with pytest.raises(Q.QmmError) as e:
        Q.qmm_nbits(d.A, d.W, d.scales, 256, 4, 48, d.zp, Q.QMM_ZP_PACKED)
    assert e.value.status == -4
    with pytest.raises(Q.QmmError) as e:
        Q.qmm_nbits(d.A, d.W, d.scales, 256, 4, 64, None, Q.QMM_ZP_PACKED)
    assert e.value.status == -1
    t.cuda.synchronize()


# --- prefill path (M > 8): A rounded to fp16 once, fp16 weights, fp32 accumulation ---

def _a_mirror(a_dtype):
    """Declared activation rounding of the matrix-core paths: fp32 and bf16 A are cast with
    the per-row power-of-two pre-scale; fp16 A is used as it is."""
    return None if a_dtype == "f16" else "f16_rows"


def _check_prefill(d, got, mrows=None, label=""):
    """Matrix-core paths: every output column against the oracle with the path's declared
    operand roundings (A: per-row pre-scaled fp16, W: fp16), every element within the
    bound of fp32 accumulation of those exact products, and, for a 16-bit output, the
    unrounded oracle at the same tolerance.  mrows: the output rows compared (all when
    None)."""
    bias, bdt = _bias_args(d)
    A = d.p["A"] if mrows is None else np.asarray(d.p["A"])[mrows]
    r = nbits_reference(O, d.p, A=A, bias=bias, bias_dtype=bdt, a_mirror=_a_mirror(d.p["a_dtype"]),
                        w_mirror="f16")
    y = host_f64(got)
    if mrows is not None:
        y = y[mrows]
    err = O.rel_l2(y, r["mirrored"])
    raw = O.rel_l2(y, r["exact"])
    say(f"  {label} relL2(mirrored)={err:.3e} relL2(unrounded)={raw:.3e}")
    assert err <= TOL[d.c_dtype], (label, err)
    if d.c_dtype != "f32":
        assert raw <= TOL[d.c_dtype], (label, raw)
    assert_elementwise(y, r["mirrored"], gamma(d.p["K"] + 2) * r["absdot"], d.c_dtype, label)
    return err


def _tile_rows(M, tile=256):
    """Output rows that meet every M tile: the first two and last two rows of each."""
    rows = set()
    for t0 in range(0, M, tile):
        t1 = min(M, t0 + tile)
        rows.update({t0, t0 + 1, t1 - 2, t1 - 1})
    return np.array(sorted(r for r in rows if 0 <= r < M))


@pytest.mark.parametrize("name", list(gen.PHI4_SHAPES))
def test_phi4_u2_prefill_full_size(name):
    """phi4-14B 2-bit shapes at M = 2048: every output column, for rows that meet every
    256-row tile."""
    K, N = gen.PHI4_SHAPES[name]
    say(f"phi4 prefill {name} K={K} N={N}")
    p = gen.nbits_problem(2048, K, N, 2, 64, seed=gen.config_seed(1, 10 + list(gen.PHI4_SHAPES).index(name)),
                          zp="f16_uniform", uniform_zp=1.5, scale_range=(0.01, 0.05))
    d = NbitsDev(p)
    got = d.run(uniform=True)
    torch().cuda.synchronize()
    _check_prefill(d, got, mrows=_tile_rows(2048), label=name)
    # the fp16 zero-point tensor path gives the same bits as the scalar path
    got_t = d.run(uniform=False)
    assert np.array_equal(host_bits(got), host_bits(got_t))


@pytest.mark.parametrize("M,K,N,bits,block,zp,a,c", [
    (9, 256, 130, 4, 64, "packed8", "f32", "f32"),
    (16, 100, 300, 2, 16, "packed", "f32", "f32"),
    (100, 5120, 257, 2, 64, "f16_uniform", "f32", "f32"),
    (300, 2880, 520, 4, 128, "packed", "f16", "f16"),
    (257, 1000, 64, 4, 32, "none", "bf16", "bf16"),
    (64, 70, 33, 2, 16, "f16", "f32", "f16"),
    (513, 4096, 300, 4, 256, "f16", "bf16", "f32"),
    # 8 < M <= 64 with blocks >= 32: the skinny kernel (16-row M tiles)
    (17, 320, 100, 2, 32, "packed", "f32", "f32"),          # last 128-code step half past Kp
    (64, 1000, 70, 4, 64, "f16", "bf16", "bf16"),           # four M tiles, ragged K and N
    (48, 4096, 4096, 4, 128, "none", "f16", "f32"),
    (40, 5120, 7680, 2, 64, "f16_uniform", "f32", "f32"),   # phi4 qkv shape, a few tokens
    (25, 2880, 33, 4, 32, "packed8", "f32", "f16"),
    (9, 64, 1, 4, 32, "packed", "f32", "f32"),              # one column, one K step
    (64, 33, 17, 2, 32, "none", "f16", "f16"),              # one-code last block
])
def test_prefill_small_shapes(M, K, N, bits, block, zp, a, c):
    say(f"prefill M={M} K={K} N={N} bits={bits} block={block} zp={zp} a={a} c={c}")
    p = gen.nbits_problem(M, K, N, bits, block, seed=11 * M + K, zp=zp, a_dtype=a, bias=(M % 2 == 1))
    d = NbitsDev(p, c_dtype=c)
    _check_prefill(d, d.run(), label=f"M={M}")


def test_prefill_exact_arithmetic_bitwise():
    """Small-integer activations and power-of-two scales make every partial sum exact,
    so the matrix-core path and the GEMV path agree bit for bit with the oracle."""
    t = torch()
    M, K, N, bits, block = 32, 512, 96, 4, 64
    p = gen.nbits_problem(M, K, N, bits, block, seed=5, zp="packed")
    rng = np.random.default_rng(6)
    p["A"] = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    p["scales"] = (2.0 ** rng.integers(-6, -2, size=p["scales"].shape)).astype(np.float16).view(np.uint16)
    d = NbitsDev(p)
    got = host_f64(d.run())
    ref = d.oracle(O)
    assert np.array_equal(got, ref)
    got1 = np.concatenate([host_f64(d.run(A=d.A[i:i + 1].contiguous())) for i in range(4)])
    assert np.array_equal(got1, ref[:4])
    t.cuda.synchronize()


@pytest.mark.parametrize("M", [32, 128], ids=["skinny", "tiles"])
@pytest.mark.parametrize("bits,zp,zval,uniform", [
    (4, "f16_uniform", 1.5, True),          # one fma per code
    (2, "f16_uniform", 0.25, True),
    (4, "f16_uniform", 100.5, True),
    (4, "f16_uniform", 300.0, True),        # |z| >= 2^8: subtract and multiply
    (4, "f16_uniform", 2.0 ** -20, True),   # a bit below 2^-15: subtract and multiply
    (4, "packed", None, False),             # integer codes: one fma per code
    (2, "f16", None, False),                # fp16 tensor: subtract and multiply
])
def test_matrix_core_weights_bit_exact(M, bits, zp, zval, uniform):
    """One-hot activation rows read the matrix-core paths' fp16 weights out exactly:
    C[m][n] = fp16(fp32((q - z) * s)) of W row n at k = m, bit for bit, whether the
    dequantization computes the product as one fma (where q - z and z * s are exact) or
    as a subtract and a multiply."""
    K, N, block = 256, 96, 32
    kw = {"uniform_zp": zval} if zval is not None else {}
    p = gen.nbits_problem(M, K, N, bits, block, seed=990 + bits + M, zp=zp, scale_range=(0.01, 0.5), **kw)
    A = np.zeros((M, K), dtype=np.float32)
    A[np.arange(M), np.arange(M)] = 1.0
    p["A"] = A
    d = NbitsDev(p)
    got = host_f64(d.run(uniform=uniform))
    torch().cuda.synchronize()
    w = O.dequant_nbits(p["W"], bits, K, block, p["scales"], p["zp"], oracle_zp_kind(O, zp)).astype(np.float64)
    want = O._round_operand(w, "f16")[:, :M].T
    assert np.array_equal(got, want), (M, bits, zp, zval, np.argwhere(got != want)[:4])


def test_prefill_repeat_bit_identical():
    p = gen.nbits_problem(512, 5120, 1024, 2, 64, seed=79, zp="f16_uniform", scale_range=(0.01, 0.05))
    d = NbitsDev(p)
    first = host_bits(d.run(uniform=True)).copy()
    out = torch().empty_like(d.run(uniform=True))
    for i in range(16):
        d.run(uniform=True, out=out)
        assert np.array_equal(host_bits(out), first), i


def test_skinny_repeat_bit_identical():
    """The skinny matrix-core path (8 < M <= 64) gives identical bits over repeated calls."""
    p = gen.nbits_problem(64, 4096, 1024, 4, 64, seed=80, zp="packed")
    d = NbitsDev(p)
    first = host_bits(d.run()).copy()
    _check_prefill(d, d.run(), label="M=64 skinny")
    out = torch().empty_like(d.run())
    for i in range(16):
        d.run(out=out)
        assert np.array_equal(host_bits(out), first), i


@pytest.mark.parametrize("M,K,a", [(40, 320, "f32"), (100, 320, "f32"), (40, 512, "bf16"),
                                   (130, 1024, "f16")])
def test_prefill_misaligned_activations_same_bits(M, K, a):
    """The A cast reads 16-byte vectors when A is 16-byte aligned and K is a multiple of
    8, else element by element: an A that starts off a 16-byte boundary (skinny and tile
    paths) gives the same bits as an aligned copy."""
    t = torch()
    p = gen.nbits_problem(M, K, 96, 4, 32, seed=81 + M, a_dtype=a, zp="packed")
    d = NbitsDev(p)
    ref = host_bits(d.run()).copy()
    n = M * K
    buf = t.empty(n + 8, dtype=d.A.dtype, device=d.A.device)
    shifted = buf[1:1 + n].view(M, K)
    shifted.copy_(d.A)
    assert shifted.data_ptr() % 16 != 0
    got = host_bits(d.run(A=shifted))
    assert np.array_equal(got, ref)
    _check_prefill(d, d.run(), label=f"M={M} K={K} {a}")


def test_empty_and_degenerate():
    t = torch()
    p = gen.nbits_problem(3, 256, 8, 4, 64, seed=9, zp="packed8", bias=True)
    d = NbitsDev(p)
    # M = 0 and N = 0: nothing to compute
    y = Q.qmm_nbits(d.A[:0], d.W, d.scales, 256, 4, 64, d.zp, Q.QMM_ZP_PACKED)
    assert y.shape == (0, 8)
    y = Q.qmm_nbits(d.A, d.W[:0], d.scales[:0], 256, 4, 64, d.zp[:0], Q.QMM_ZP_PACKED)
    assert y.shape == (3, 0)
    # K = 1: one code of a ragged block; every weight row is (q - 8) * s
    p1 = gen.nbits_problem(2, 1, 8, 4, 64, seed=10, zp="packed8", bias=True)
    d1 = NbitsDev(p1)
    assert O.rel_l2(host_f64(d1.run()), d1.oracle(O)) <= TOL["f32"]
    # M = 20 with K = 1 on the prefill path
    p2 = gen.nbits_problem(20, 1, 8, 2, 16, seed=11, zp="packed")
    d2 = NbitsDev(p2)
    assert O.rel_l2(host_f64(d2.run()), d2.oracle(O, a_round="f16_rows", w_round="f16")) <= TOL["f32"]
    t.cuda.synchronize()


# --- activation outliers and range ----------------------------------------------

def _store_act(x64, a_dtype):
    """fp64 activations -> the storage of a_dtype (fp32 array or 16-bit patterns)."""
    t = torch()
    if a_dtype == "f32":
        return x64.astype(np.float32)
    if a_dtype == "f16":
        return x64.astype(np.float16).view(np.uint16)
    return t.from_numpy(x64.astype(np.float32)).to(t.bfloat16).view(t.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("bits,zp,a,at_zp", [
    (2, "packed", "f32", True), (4, "packed", "f32", True), (2, "none", "bf16", True),
    (4, "none", "f16", True), (2, "f16_uniform", "f32", False), (4, "packed", "f32", False),
])
def test_gemv_activation_outliers(M, bits, zp, a, at_zp):
    """One activation of magnitude 1e3..1e4 in every 64-value group ("massive
    activations"), at the 1e-5 gate of an fp32 output.  at_zp: the weight code at each
    outlier equals its block's zero point, so the outliers contribute nothing and the
    output is made of the ordinary activations alone."""
    K, N, block = 5120, 384, 64
    say(f"gemv outliers M={M} bits={bits} zp={zp} a={a} at_zp={at_zp}")
    p = gen.nbits_problem(M, K, N, bits, block, seed=300 + 7 * bits + M + at_zp, zp=zp, uniform_zp=1.5,
                          scale_range=(0.01, 0.05))
    rng = np.random.default_rng(301 + M)
    x = rng.standard_normal((M, K))
    pos = np.arange(0, K, 64) + rng.integers(0, 64, size=K // 64)
    x[:, pos] = rng.uniform(1e3, 1e4, size=(M, len(pos))) * rng.choice([-1.0, 1.0], size=(M, len(pos)))
    p["A"] = _store_act(x, a)
    p["a_dtype"] = a
    if at_zp:
        q = O.unpack_codes(p["W"], bits, K, block).astype(np.int64)
        nblk = gen.nblocks(K, block)
        z = O.zero_points_f64(p["zp"], {"packed": O.ZP_PACKED, "none": O.ZP_NONE}[zp], bits, N, nblk)
        q[:, pos] = z[:, pos // block].astype(np.int64)
        p["W"] = O.pack_codes(q.astype(np.uint8), bits, block)
    d = NbitsDev(p, c_dtype="f32")
    _check(d, d.run(uniform=(zp == "f16_uniform")), label=f"outliers M={M}")


@pytest.mark.parametrize("M,K,N,a,c", [
    (16, 4096, 512, "bf16", "bf16"),   # skinny kernel
    (40, 1000, 200, "f32", "f32"),     # skinny kernel, K not a multiple of 64
    (200, 2048, 300, "bf16", "f32"),   # 256 x 256 tiles
    (300, 640, 256, "f32", "f32"),
])
def test_matrix_core_activation_range(M, K, N, a, c):
    """Rows whose values pass the fp16 range (1e5) or lie below its normal range (1e-6,
    3e-9), and a row with one value past it: the per-row power-of-two pre-scale of the
    activation cast keeps every row finite and near its unrounded result."""
    say(f"activation range M={M} K={K} N={N} a={a}")
    p = gen.nbits_problem(M, K, N, 4, 64, seed=310 + M, zp="packed", a_dtype="f32", bias=True)
    x = np.asarray(p["A"], dtype=np.float64)
    x[0] *= 1e5
    x[1] *= 1e-6
    x[2] *= 3e-9
    x[3, 7] = 7e4
    p["A"] = _store_act(x, a)
    p["a_dtype"] = a
    d = NbitsDev(p, c_dtype=c)
    y = d.run()
    torch().cuda.synchronize()
    got = host_f64(y)
    assert np.all(np.isfinite(got))
    _check_prefill(d, y, label=f"range M={M}")
    bias, bdt = _bias_args(d)
    r = nbits_reference(O, d.p, bias=bias, bias_dtype=bdt)
    for m in range(4):
        err = O.rel_l2(got[m], r["exact"][m])
        say(f"  row {m}: relL2(unrounded)={err:.3e}")
        assert err <= 2e-3, (m, err)


def test_first_call_of_new_shape_under_capture():
    """The first call of a shape no other test uses, made while the stream is captured:
    nothing is timed (the capture would fail on the timing's synchronization), the
    default tiling runs, and every replay and the later timed eager call give the same
    bits."""
    t = torch()
    p = gen.nbits_problem(2, 3072, 777, 4, 64, seed=320, zp="packed", bias=True)
    d = NbitsDev(p)
    out = t.empty((2, 777), dtype=t.float32, device="cuda")
    t.cuda.synchronize()
    cap = t.cuda.Stream()
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(cap):
        with t.cuda.graph(g, stream=cap):
            d.run(out=out)
    t.cuda.synchronize()
    reps = []
    for _ in range(3):
        out.zero_()
        g.replay()
        t.cuda.synchronize()
        reps.append(host_bits(out).copy())
    eager = host_bits(d.run()).copy()   # first uncaptured call: times the candidates
    for r_ in reps:
        assert np.array_equal(r_, eager)
    _check(d, d.run(), label="after capture")


# --- 3-bit and signed 8-bit weights ([P1] kernel unit-test leaves Wu3, Wi8) ------

@pytest.mark.parametrize("bits,block,K,zp", [
    (3, 32, 200, "packed"), (3, 64, 5120, "f16"), (3, 128, 300, "none"), (3, 256, 1000, "packed8"),
    (8, 16, 70, "packed"), (8, 32, 2880, "none"), (8, 64, 512, "f16"), (8, 128, 300, "f16_uniform"),
])
@pytest.mark.parametrize("out", ["f32", "f16"])
def test_dequant_wide_codes_bit_exact(bits, block, K, zp, out):
    say(f"dequant bits={bits} block={block} K={K} zp={zp} out={out}")
    t = torch()
    p = gen.nbits_problem(1, K, 96, bits, block, seed=500 + K + bits, zp=zp)
    d = NbitsDev(p)
    got = Q.qmm_dequantize_nbits(d.W, d.scales, K, bits, block, d.zp, gpu_kind(zp),
                                 out_dtype=t.float32 if out == "f32" else t.float16)
    w = O.dequant_nbits(p["W"], bits, K, block, p["scales"], p["zp"], oracle_zp_kind(O, zp))
    if out == "f32":
        assert np.array_equal(host_bits(got).view(np.uint32), w.view(np.uint32))
    else:
        assert np.array_equal(host_bits(got).view(np.uint16), O.to_f16(w).view(np.uint16))


WIDE_SHAPES = [(1000, 300, 32, "packed"), (2880, 257, 64, "f16"), (4096, 520, 128, "none")]


@pytest.mark.parametrize("shape", range(len(WIDE_SHAPES)))
@pytest.mark.parametrize("M", [1, 5, 33, 300])
@pytest.mark.parametrize("bits", [3, 8])
@pytest.mark.parametrize("leaf", ["f16", "f32"])
def test_wide_codes_leaf_grid(leaf, bits, M, shape):
    """The page's leaves X{fp16, fp32} x W{u3, i8} with the output in the activation type:
    GEMV (M <= 8), skinny matrix-core kernel (8 < M <= 64) and 256 x 256 tiles."""
    K, N, block, zp = WIDE_SHAPES[shape]
    say(f"leaf X{leaf} W{'u3' if bits == 3 else 'i8'} M={M} K={K} N={N} block={block} zp={zp}")
    p = gen.nbits_problem(M, K, N, bits, block, seed=510 + 7 * M + K + bits, zp=zp, a_dtype=leaf,
                          bias=(M % 2 == 1))
    d = NbitsDev(p, c_dtype=leaf)
    y = d.run()
    if M > 8:
        _check_prefill(d, y, label=f"M={M}")
    else:
        _check(d, y, label=f"M={M}")


def test_wide_codes_repeat_and_candidates():
    """3-bit GEMV: every tiling candidate gives the same bits, and repeated calls too."""
    p = gen.nbits_problem(3, 4096, 1000, 3, 64, seed=530, zp="packed")
    d = NbitsDev(p)
    outs = []
    try:
        for c in range(Q.num_candidates(Q.ENTRY_NBITS)):
            Q.set_tuning(2, c)
            outs.append(host_bits(d.run()).copy())
    finally:
        Q.set_tuning(0, 0)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    for _ in range(8):
        assert np.array_equal(host_bits(d.run()), outs[0])
