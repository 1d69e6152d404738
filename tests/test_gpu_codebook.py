"""GPU parity of qmm_codebook4 / qmm_dequantize_codebook4 against the oracle."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import inputs as gen
from gemm_qmm_nbits_amd import qmm as Q
from oracle import qmm_oracle as O

from gpu_util import TOL, dev, dev_act, host_bits, host_f64, sample_rows, say, torch

pytestmark = pytest.mark.gpu


def cb_matrix_path(M, block, out_dtype):
    """Whether qmm_codebook4 takes a matrix-core path: M > 8, or 4 <= M <= 8 with a
    16-bit output and blocks of at least 32 codes (the skinny kernel)."""
    t = torch()
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

    def check(self, y, rows=None, label=""):
        """GEMV path: against the exact oracle.  Matrix-core path: against the oracle
        with its declared operand roundings (A and W to fp16); the error against the exact
        oracle is printed for information."""
        got = host_f64(y)
        if rows is not None:
            got = got[:, rows]
        tol = TOL[self.p["a_dtype"]]
        if cb_matrix_path(self.p["A"].shape[0], self.p["block"], y.dtype):
            err = O.rel_l2(got, self.oracle(rows=rows, a_round="f16", w_round="f16"))
            raw = O.rel_l2(got, self.oracle(rows=rows))
            say(f"  {label} relL2(mirrored)={err:.3e} relL2(exact)={raw:.3e}")
        else:
            err = O.rel_l2(got, self.oracle(rows=rows))
            say(f"  {label} relL2={err:.3e}")
        assert err <= tol, (label, err)


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
    rows = sample_rows(N, 2048, seed=N + M)
    d.check(y, rows=rows, label=f"{name} M={M}")


@pytest.mark.parametrize("M", [1, 3, 8])
def test_codebook_ragged_bias(M):
    p = gen.codebook_problem(M, 1000, 300, seed=55 + M, a_dtype="bf16", block=32, bias=True)
    d = CbDev(p)
    d.check(d.run(), label=f"M={M}")


@pytest.mark.parametrize("M,out", [(4, "same"), (5, "same"), (7, "same"), (8, "same"),
                                   (4, "f32"), (8, "f32")])
def test_codebook_small_m_paths(M, out):
    """4 <= M <= 8: a 16-bit output takes the skinny kernel (gate: the oracle with fp16
    operands; the reduction is split at this width); an fp32 output keeps the GEMV
    (gate: the exact oracle at the fp32 tolerance)."""
    t = torch()
    p = gen.codebook_problem(M, 4096, 1024, seed=58 + M, a_dtype="bf16", block=64,
                             bias=(out == "same"))
    d = CbDev(p)
    if out == "f32":
        y = Q.qmm_codebook4(d.A, d.W, d.absmax, d.cb, p["K"], p["block"], None,
                            out_dtype=t.float32)
        assert not cb_matrix_path(M, p["block"], y.dtype)
        err = O.rel_l2(host_f64(y), d.oracle())
        say(f"  M={M} fp32 out relL2={err:.3e}")
        assert err <= TOL["f32"], err
    else:
        y = d.run()
        assert cb_matrix_path(M, p["block"], y.dtype)
        d.check(y, label=f"M={M} bf16 out")


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
    assert not cb_matrix_path(M, block, y.dtype)
    err = O.rel_l2(host_f64(y), d.oracle())
    say(f"  M={M} K={K} N={N} block={block} {out}: relL2={err:.3e}")
    assert err <= (TOL["f32"] if out == "f32" else TOL["bf16"]), err


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
