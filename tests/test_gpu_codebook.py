"""GPU parity of qmm_codebook4 / qmm_dequantize_codebook4 against the oracle."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import inputs as gen
from gemm_qmm_nbits_amd import qmm as Q
from oracle import qmm_oracle as O

from gpu_util import TOL, assert_elementwise, column_chunks, dev, dev_act, gamma, host_bits, host_f64, say, torch

pytestmark = pytest.mark.gpu


def cb_matrix_path(M, K, N, block, out_dtype):
    """Whether qmm_codebook4 takes a matrix-core path: M > 8, or 4 <= M <= 8 with a
    16-bit output and blocks of at least 32 codes (the skinny kernel), except M = 4 on
    at most 2^24 codes (the GEMV's four-row form)."""
    t = torch()
    if M == 4 and N * K <= 1 << 24:
        return False
    return M > 8 or (M >= 4 and block >= 32 and out_dtype in (t.float16, t.bfloat16))


class CbDev:
    def __init__(self, p):
        t = torch()
        self.p = p
        self.A = dev_act(p["A"], p["a_dtype"])
        self.W = dev(p["W"])
        self.absmax = dev(p["absmax"])
        self.cb = dev(p["codebook"])
        td = {"f32": t.float32, "f16": t.float16, "bf16": t.bfloat16}[p["a_dtype"]]
        self.bias = (t.from_numpy(np.asarray(p["bias"], dtype=np.uint16).view(np.int16)).cuda().view(td)
                     if p["bias"] is not None else None)

    def run(self, out=None):
        p = self.p
        return Q.qmm_codebook4(self.A, self.W, self.absmax, self.cb, p["K"], p["block"], self.bias,
                               out=out)

    def oracle(self, rows=None, w_round=None, a_round=None):
        p = self.p
        return O.qmm_codebook4(p["A"], p["a_dtype"], p["W"], p["K"], p["block"], p["absmax"],
                               p["codebook"], bias=p["bias"], rows=rows, w_round=w_round,
                               a_round=a_round)

    def reference(self, a_round=None, w_round=None):
        """Whole-width oracle, one column chunk at a time: (exact, mirrored, sum |a'||w'|)."""
        p = self.p
        a = O.activations_f64(p["A"], p["a_dtype"])
        am = O._round_operand(a, a_round) if a_round else a
        b = None if p["bias"] is None else O.activations_f64(p["bias"], p["a_dtype"])
        N = p["N"]
        exact = np.zeros((a.shape[0], N))
        mirr = np.zeros((a.shape[0], N))
        absdot = np.zeros((a.shape[0], N))
        for cols in column_chunks(N):
            w = O.dequant_codebook4(np.asarray(p["W"])[cols], p["K"], p["block"],
                                    np.asarray(p["absmax"])[cols], p["codebook"]).astype(np.float64)
            wm = O._round_operand(w, w_round) if w_round else w
            bc = None if b is None else b[cols]
            exact[:, cols] = O.matmul_f64(a, w, bc)
            mirr[:, cols] = O.matmul_f64(am, wm, bc)
            absdot[:, cols] = np.abs(am) @ np.abs(wm).T
        return exact, mirr, absdot

    def check(self, y, label=""):
        """Every output column.  GEMV path: against the exact oracle, every element within
        the bound of fp32 accumulation.  Matrix-core path: against the oracle with its
        declared operand roundings (A: per-row pre-scaled fp16 unless already fp16, W: fp16),
        every element within the bound of fp32 accumulation of those products, and for a
        16-bit output also against the unrounded oracle at the same tolerance."""
        got = host_f64(y)
        out_dt = {torch().float32: "f32", torch().float16: "f16", torch().bfloat16: "bf16"}[y.dtype]
        tol = TOL[out_dt]
        K = self.p["K"]
        if cb_matrix_path(self.p["A"].shape[0], self.p["K"], self.p["N"], self.p["block"], y.dtype):
            a_round = None if self.p["a_dtype"] == "f16" else "f16_rows"
            exact, mirr, absdot = self.reference(a_round=a_round, w_round="f16")
            err = O.rel_l2(got, mirr)
            raw = O.rel_l2(got, exact)
            say(f"  {label} relL2(mirrored)={err:.3e} relL2(exact)={raw:.3e}")
            assert err <= tol, (label, err)
            if out_dt != "f32":
                assert raw <= tol, (label, raw)
            assert_elementwise(got, mirr, gamma(K + 2) * absdot, out_dt, label)
        else:
            exact, _, absdot = self.reference()
            err = O.rel_l2(got, exact)
            say(f"  {label} relL2={err:.3e}")
            assert err <= tol, (label, err)
            assert_elementwise(got, exact, gamma(K + 4) * absdot, out_dt, label)


@pytest.mark.parametrize("out", ["f32", "f16"])
@pytest.mark.parametrize("K,block", [(4096, 64), (1536, 64), (200, 32), (300, 256)])
def test_dequant_codebook_bit_exact(K, block, out):
    t = torch()
    p = gen.codebook_problem(1, K, 77, seed=K + block, block=block)
    d = CbDev(p)
    got = Q.qmm_dequantize_codebook4(d.W, d.absmax, d.cb, K, block,
                                     out_dtype=t.float32 if out == "f32" else t.float16)
    w = O.dequant_codebook4(p["W"], K, block, p["absmax"], p["codebook"])
    if out == "f32":
        assert np.array_equal(host_bits(got).view(np.uint32), w.view(np.uint32))
    else:
        assert np.array_equal(host_bits(got).view(np.uint16), O.to_f16(w).view(np.uint16))


@pytest.mark.parametrize("a_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M", gen.CODEBOOK_M)
@pytest.mark.parametrize("name", list(gen.CODEBOOK_SHAPES))
def test_codebook_config_shapes(name, M, a_dtype):
    """16-entry codebook skinny GEMM at the four shapes, M in {1, 4, 16, 64}, bf16/fp16."""
    K, N = gen.CODEBOOK_SHAPES[name]
    say(f"codebook {name} K={K} N={N} M={M} {a_dtype}")
    idx = list(gen.CODEBOOK_SHAPES).index(name)
    p = gen.codebook_problem(M, K, N, seed=gen.config_seed(2, 10 * idx + M), a_dtype=a_dtype)
    d = CbDev(p)
    y = d.run()
    d.check(y, label=f"{name} M={M}")


@pytest.mark.parametrize("M", [1, 3, 8])
def test_codebook_ragged_bias(M):
    p = gen.codebook_problem(M, 1000, 300, seed=55 + M, a_dtype="bf16", block=32, bias=True)
    d = CbDev(p)
    d.check(d.run(), label=f"M={M}")


@pytest.mark.parametrize("M,N,out", [(4, 1024, "same"), (4, 4096, "same"), (4, 4160, "same"), (5, 1024, "same"),
                                     (7, 1024, "same"), (8, 1024, "same"), (4, 4160, "f32"),
                                     (8, 1024, "f32")])
def test_codebook_small_m_paths(M, N, out):
    """4 <= M <= 8: a 16-bit output takes the skinny kernel (gate: the oracle with fp16
    operands; the reduction is split at this width), except M = 4 on at most 2^24 codes,
    which the GEMV keeps; an fp32 output keeps the GEMV (gate: the exact oracle at the
    fp32 tolerance)."""
    t = torch()
    p = gen.codebook_problem(M, 4096, N, seed=58 + M + N, a_dtype="bf16", block=64,
                             bias=(out == "same"))
    d = CbDev(p)
    if out == "f32":
        y = Q.qmm_codebook4(d.A, d.W, d.absmax, d.cb, p["K"], p["block"], d.bias,
                            out_dtype=t.float32)
        assert not cb_matrix_path(M, p["K"], N, p["block"], y.dtype)
        d.check(y, label=f"M={M} N={N} fp32 out")
    else:
        y = d.run()
        assert cb_matrix_path(M, p["K"], N, p["block"], y.dtype) == (M > 4 or N * p["K"] > 1 << 24)
        d.check(y, label=f"M={M} N={N} bf16 out")


@pytest.mark.parametrize("M,K,N,block,out", [
    (1, 20480, 300, 64, "same"),   # A does not fit in LDS: the general kernel, K in slices
    (2, 20480, 77, 64, "f32"),     # the same with two A rows and an fp32 output
    (4, 12288, 64, 64, "f32"),     # four A rows, six slices
    (1, 2000, 129, 16, "same"),    # 16-code blocks: two absmax values per chunk (general kernel)
    (1, 4096, 1, 64, "same"),      # streaming form, one output row
    (1, 64, 5, 64, "same"),        # streaming form, K of two chunks (most lanes idle)
    (3, 4096, 1000, 128, "f32"),   # streaming form, three A rows, 128-code blocks
])
def test_codebook_gemv_forms(M, K, N, block, out):
    """M <= 8 GEMV paths the configuration shapes do not reach, against the exact oracle."""
    t = torch()
    p = gen.codebook_problem(M, K, N, seed=59 + K + N, a_dtype="bf16", block=block,
                             bias=(out == "same"))
    d = CbDev(p)
    od = None if out == "same" else t.float32
    y = Q.qmm_codebook4(d.A, d.W, d.absmax, d.cb, K, block, d.bias, out_dtype=od)
    assert not cb_matrix_path(M, K, N, block, y.dtype)
    d.check(y, label=f"M={M} K={K} N={N} block={block} {out}")


def test_codebook_repeat_bit_identical():
    p = gen.codebook_problem(4, 4096, 4096, seed=56, a_dtype="f16")
    d = CbDev(p)
    first = host_bits(d.run()).copy()
    out = torch().empty_like(d.run())
    for i in range(128):
        d.run(out=out)
        assert np.array_equal(host_bits(out), first), i


@pytest.mark.parametrize("M,K,N,block,a_dtype", [
    (9, 1000, 300, 32, "bf16"),     # ragged K (last stage half padding), ragged N tile
    (33, 4096, 257, 64, "f16"),
    (300, 200, 64, 256, "bf16"),    # one block longer than K, two M tiles
    (64, 96, 5, 32, "f16"),         # skinny path: ragged N, K of three blocks
    (16, 4096, 1024, 64, "bf16"),   # skinny path with the reduction split
])
def test_codebook_matrix_core_ragged(M, K, N, block, a_dtype):
    """M > 8 runs the matrix-core path; ragged M, N, K and a bias."""
    p = gen.codebook_problem(M, K, N, seed=57 + M, a_dtype=a_dtype, block=block, bias=True)
    d = CbDev(p)
    d.check(d.run(), label=f"M={M} K={K} N={N}")


# --- nested (double-quantized) absmax ----------------------------------------------

def _nested_dev(na):
    t = torch()
    return {"codes": dev(na["codes"]), "table": dev(na["table"]), "scales": dev(na["scales"]),
            "offset": float(na["offset"]), "group": na["group"]}


@pytest.mark.parametrize("group", [256, 64, 1])
def test_nested_absmax_decode_bit_exact(group):
    rng = np.random.default_rng(700 + group)
    na = gen.nested_absmax_inputs(rng, 4096, 64, group=group)
    got = Q.qmm_dequantize_absmax_nested(_nested_dev(na), 4096 * 64)
    want = O.nested_absmax(na["codes"], na["table"], na["scales"], na["offset"], group)
    assert np.array_equal(host_bits(got).view(np.uint32), want.ravel().view(np.uint32))


@pytest.mark.parametrize("M", [1, 4, 16, 64])
@pytest.mark.parametrize("name", ["square", "moe_down"])
def test_codebook_nested_absmax(name, M):
    """The codebook matmul with nested absmax equals, bit for bit, the plain entry on the
    decoded absmax, and the oracle on the oracle's decoded absmax within the gate."""
    K, N = gen.CODEBOOK_SHAPES[name]
    say(f"codebook nested {name} M={M}")
    p = gen.codebook_problem(M, K, N, seed=710 + M, a_dtype="bf16")
    rng = np.random.default_rng(711 + M)
    na = gen.nested_absmax_inputs(rng, N, K // 64)
    am = O.nested_absmax(na["codes"], na["table"], na["scales"], na["offset"], na["group"])
    p["absmax"] = am
    d = CbDev(p)
    y = Q.qmm_codebook4_nested(d.A, d.W, _nested_dev(na), d.cb, K, 64)
    plain = d.run()
    assert np.array_equal(host_bits(y), host_bits(plain))
    d.check(y, label=f"nested {name} M={M}")
