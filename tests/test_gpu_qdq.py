"""GPU parity of the activation quantization ops and the fused quantized SwiGLU against
the oracle (bit-exact codes and values), and of the fused ops against the unfused chain
run on the device."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import qmm as Q
from oracle import qmm_oracle as O

from gpu_util import dev, host_bits, say, torch

pytestmark = pytest.mark.gpu


def _x(n, seed, scale=1.5):
    """fp32 activations with specials: zeros, signed zeros, NaN, infinities, huge values."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * scale).astype(np.float32)
    sp = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 3e38, -3e38, 1e-40], dtype=np.float32)
    x[: len(sp)] = sp
    return x


def _to(x32, dt):
    """fp32 values -> a device tensor of dtype dt, and the stored values as fp32."""
    t = torch()
    td = {"f32": t.float32, "f16": t.float16, "bf16": t.bfloat16}[dt]
    xt = t.from_numpy(x32).to(td).cuda()
    return xt, xt.float().cpu().numpy()


def _bits_of(y, dt):
    return host_bits(y).view(np.uint32 if dt == "f32" else np.uint16)


def _round_out(v32, dt):
    """fp32 results -> the bit patterns of the output dtype (nearest, ties to even)."""
    if dt == "f32":
        return np.asarray(v32, dtype=np.float32).view(np.uint32)
    if dt == "f16":
        return O.to_f16(v32).view(np.uint16)
    return O.f32_to_bf16_bits(v32)


PARAMS = {8: [(np.float32(0.0123), 128), (np.float32(2.0 ** -5), 0), (np.float32(0.7), 255)],
          16: [(np.float32(1.0 / 4096), 32768), (np.float32(3.1e-4), 1000), (np.float32(0.25), 65535)]}


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [8, 16])
def test_quantize_dequantize_fake_quantize(bits, dt):
    """Q, DQ and the fused Q -> DQ against the oracle bit for bit; the fused op equals the
    device chain DQ(Q(x)) bit for bit."""
    t = torch()
    n = 1_000_003
    for i, q in enumerate(PARAMS[bits]):
        xt, x32 = _to(_x(n, 600 + 3 * bits + i), dt)
        codes = Q.quantize_linear(xt, q, bits)
        want_q = O.quantize_linear(x32, q[0], q[1], bits)
        got_q = codes.cpu().numpy().astype(np.int64)
        assert np.array_equal(got_q, want_q.astype(np.int64)), (bits, dt, q)
        y = Q.dequantize_linear(codes, q, bits, out_dtype=xt.dtype)
        assert np.array_equal(_bits_of(y, dt), _round_out(O.dequantize_linear(want_q, q[0], q[1]), dt))
        fq = Q.fake_quantize(xt, q, bits)
        assert np.array_equal(_bits_of(fq, dt), _round_out(O.fake_quantize(x32, q[0], q[1], bits), dt))
        assert np.array_equal(_bits_of(fq, dt), _bits_of(y, dt))
    t.cuda.synchronize()


@pytest.mark.parametrize("bits", [8, 16])
def test_qsigmoid_and_qmul(bits):
    t = torch()
    rng = np.random.default_rng(610 + bits)
    qmax = (1 << bits) - 1
    n = 300_001
    codes = rng.integers(0, qmax + 1, size=n).astype(O.code_dtype(bits))
    codes[:qmax + 1 if bits == 8 else 0] = np.arange(qmax + 1 if bits == 8 else 0)  # every code (uint8)
    dc = dev(codes.view(np.int16) if bits == 16 else codes).view(t.uint16 if bits == 16 else t.uint8)
    qi, qo = (np.float32(8.0 / qmax), 1 << (bits - 1)), (np.float32(1.0 / qmax), 0)
    got = Q.qsigmoid(dc, qi, qo, bits).cpu().numpy().astype(np.int64)
    want = O.qsigmoid(codes, qi[0], qi[1], qo[0], qo[1], bits).astype(np.int64)
    assert np.array_equal(got, want)
    codes_b = rng.integers(0, qmax + 1, size=n).astype(O.code_dtype(bits))
    db = dev(codes_b.view(np.int16) if bits == 16 else codes_b).view(t.uint16 if bits == 16 else t.uint8)
    qa, qb, qc = (np.float32(0.031), 100), (np.float32(0.017), 9), (np.float32(0.0093), 40)
    got = Q.qmul(dc, qa, db, qb, qc, bits).cpu().numpy().astype(np.int64)
    want = O.qmul(codes, qa[0], qa[1], codes_b, qb[0], qb[1], qc[0], qc[1], bits).astype(np.int64)
    assert np.array_equal(got, want)


SWIGLU_Q = {8: [(np.float32(6.0 / 255), 128), (np.float32(1.0 / 255), 0), (np.float32(7.0 / 255), 128),
                (np.float32(6.0 / 255), 128), (np.float32(9.0 / 255), 128)],
            16: [(np.float32(12.0 / 65535), 32768), (np.float32(1.0 / 65535), 0),
                 (np.float32(14.0 / 65535), 32768), (np.float32(12.0 / 65535), 32768),
                 (np.float32(40.0 / 65535), 32768)]}


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [8, 16])
def test_qswiglu_fused_equals_chain(bits, dt):
    """The fused quantized SwiGLU equals the chain of unfused device ops (Q(gate),
    qsigmoid, qmul, Q(up), qmul, DQ) bit for bit, and the oracle's chain bit for bit."""
    t = torch()
    n = 2_000_005
    qp = SWIGLU_Q[bits]
    gate, g32 = _to(_x(n, 620 + bits, 2.0), dt)
    up, u32 = _to(_x(n, 630 + bits, 2.0), dt)
    y = Q.qswiglu(gate, up, qp, bits)
    g = Q.quantize_linear(gate, qp[0], bits)
    s = Q.qsigmoid(g, qp[0], qp[1], bits)
    m = Q.qmul(g, qp[0], s, qp[1], qp[2], bits)
    u = Q.quantize_linear(up, qp[3], bits)
    h = Q.qmul(m, qp[2], u, qp[3], qp[4], bits)
    chain = Q.dequantize_linear(h, qp[4], bits, out_dtype=gate.dtype)
    t.cuda.synchronize()
    assert np.array_equal(_bits_of(y, dt), _bits_of(chain, dt))
    want = O.qswiglu(g32, u32, qp, bits)
    got = _bits_of(y, dt)
    exp = _round_out(want, dt)
    bad = np.nonzero(got != exp)[0]
    say(f"  qswiglu bits={bits} {dt}: {len(bad)} mismatches of {n}")
    assert len(bad) == 0, (bad[:5], got[bad[:5]], exp[bad[:5]])


def test_quantization_refusals():
    t = torch()
    x = t.zeros(16, device="cuda")
    with pytest.raises(Q.QmmError) as e:
        Q.quantize_linear(x, (1.0, 0), 4)
    assert e.value.status == -3
    for bad in ((0.0, 0), (-1.0, 0), (float("nan"), 0), (float("inf"), 0), (1.0, 256), (1.0, -1)):
        with pytest.raises(Q.QmmError) as e:
            Q.quantize_linear(x, bad, 8)
        assert e.value.status == -10, bad
    with pytest.raises(Q.QmmError) as e:
        Q.qswiglu(x, x, [(1.0, 0)] * 4 + [(1.0, 70000)], 16)
    assert e.value.status == -10
    assert Q.quantize_linear(x[:0], (1.0, 0), 8).numel() == 0
