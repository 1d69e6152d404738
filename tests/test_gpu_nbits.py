"""GPU parity of qmm_nbits / qmm_dequantize_nbits / qmm_fp16_uniform_value against the oracle."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import inputs as gen
from gemm_qmm_nbits_amd import qmm as Q
from oracle import qmm_oracle as O

from gpu_util import TOL, NbitsDev, dev, host_bits, host_f64, oracle_zp_kind, sample_rows, say, torch

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

def _check(d, got, rows=None, label=""):
    ref = d.oracle(O, rows=rows)
    y = host_f64(got)
    if rows is not None:
        y = y[:, rows]
    err = O.rel_l2(y, ref)
    say(f"  {label} relL2={err:.3e} (tol {TOL[d.c_dtype]:.0e})")
    assert err <= TOL[d.c_dtype], (label, err)


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
    rows = None if N <= 8192 else sample_rows(N, 1024, seed=N)
    _check(d, got_u, rows=rows, label=name)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 11])
@pytest.mark.parametrize("bits,block,K,N,zp,a,c", [
    (2, 64, 1000, 300, "packed", "f32", "f32"),
    (4, 32, 2880, 257, "packed", "f16", "f16"),
    (4, 128, 2880, 190, "none", "bf16", "bf16"),
    (2, 16, 512, 130, "f16", "f32", "f16"),
    (2, 16, 70, 33, "packed", "f32", "f32"),     # 20-byte rows: generic kernel
    (4, 256, 1536, 64, "f16", "bf16", "f32"),
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
        Q.qmm_nbits(d.A, d.W, d.scales, 256, 3, 64, d.zp, Q.QMM_ZP_PACKED)
    assert e.value.status == -3
    with pytest.raises(Q.QmmError) as e:
        Q.qmm_nbits(d.A, d.W, d.scales, 256, 4, 48, d.zp, Q.QMM_ZP_PACKED)
    assert e.value.status == -4
    with pytest.raises(Q.QmmError) as e:
        Q.qmm_nbits(d.A, d.W, d.scales, 256, 4, 64, None, Q.QMM_ZP_PACKED)
    assert e.value.status == -1
    t.cuda.synchronize()


# --- prefill path (M > 8): A rounded to fp16 once, fp16 weights, fp32 accumulation ---

def _check_prefill(d, got, rows=None, label=""):
    """Gate against the oracle with the path's declared operand roundings (A and W
    to fp16); the error against the unrounded oracle is printed for information."""
    y = host_f64(got)
    if rows is not None:
        y = y[:, rows]
    ref = d.oracle(O, rows=rows, a_round="f16", w_round="f16")
    err = O.rel_l2(y, ref)
    raw = O.rel_l2(y, d.oracle(O, rows=rows))
    say(f"  {label} relL2(mirrored)={err:.3e} relL2(unrounded)={raw:.3e}")
    assert err <= TOL[d.c_dtype], (label, err)
    return err


@pytest.mark.parametrize("name", list(gen.PHI4_SHAPES))
def test_phi4_u2_prefill_full_size(name):
    """phi4-14B 2-bit shapes at M = 2048 (full size; oracle on sampled output columns)."""
    K, N = gen.PHI4_SHAPES[name]
    say(f"phi4 prefill {name} K={K} N={N}")
    p = gen.nbits_problem(2048, K, N, 2, 64, seed=gen.config_seed(1, 10 + list(gen.PHI4_SHAPES).index(name)),
                          zp="f16_uniform", uniform_zp=1.5, scale_range=(0.01, 0.05))
    d = NbitsDev(p)
    got = d.run(uniform=True)
    torch().cuda.synchronize()
    rows = sample_rows(N, 192, seed=N + 1)
    _check_prefill(d, got, rows=rows, label=name)
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
    assert O.rel_l2(host_f64(d2.run()), d2.oracle(O, a_round="f16", w_round="f16")) <= TOL["f32"]
    t.cuda.synchronize()
