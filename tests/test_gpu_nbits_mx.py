"""The matrix-core form of the 2-bit GEMV (tuning candidate 3): the same bits as
the v_dot8 kernel on every shape it serves, and parity with the oracle on sampled
output columns."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import inputs as gen
from gemm_qmm_nbits_amd import qmm as Q
from oracle import qmm_oracle as O

from gpu_util import TOL, NbitsDev, host_bits, host_f64, sample_rows, say, torch

pytestmark = pytest.mark.gpu

MX_CANDIDATES = (3,)


@pytest.mark.parametrize("K,N,block,zp,a,c,bias,outliers", [
    # 16 lanes per row in the v_dot8 kernel, rows not a multiple of 16 or 32
    (5120, 14000, 64, "f16_uniform", "f32", "f32", False, False),
    # random packed zero points, bias, outliers, fp16 in and out
    (5120, 16400, 64, "packed", "f16", "f16", True, True),
    # fp16 zero-point tensor, bf16 activations, 32 lanes per row (one round of 8 pairs)
    (2048, 20000, 64, "f16", "bf16", "bf16", False, False),
    # packed zero point 2, bias, rows a multiple of 16
    (5120, 20000, 64, "packed8", "f32", "f32", True, False),
    # 12 pairs (three rounds), uniform zero point, fp16 activations, fp32 output
    (3072, 20000, 64, "f16_uniform", "f16", "f32", False, False),
    # 32 lanes per row, three rounds, outliers, no zero point
    (6144, 9000, 64, "none", "f32", "f32", False, True),
    # the lm_head shape, uniform zero point
    (5120, 100352, 64, "f16_uniform", "f32", "f32", False, False),
])
def test_matrix_core_gemv_same_bits(K, N, block, zp, a, c, bias, outliers):
    say(f"matrix-core gemv K={K} N={N} block={block} zp={zp} a={a} c={c} bias={bias} outliers={outliers}")
    assert Q.nbits_gemv_matrix_core_form(1, K, N, 2, block)
    p = gen.nbits_problem(1, K, N, 2, block, seed=900 + K % 97 + N % 89, a_dtype=a, zp=zp, uniform_zp=1.5,
                          bias=bias, scale_range=(0.01, 0.05))
    if outliers:
        rng = np.random.default_rng(901)
        x = rng.standard_normal((1, K))
        pos = np.arange(0, K - 63, 64) + rng.integers(0, 64, size=K // 64)
        x[:, pos] = rng.uniform(1e3, 1e4, size=(1, len(pos))) * rng.choice([-1.0, 1.0], size=(1, len(pos)))
        t = torch()
        if a == "f32":
            p["A"] = x.astype(np.float32)
        elif a == "f16":
            p["A"] = x.astype(np.float16).view(np.uint16)
        else:
            p["A"] = t.from_numpy(x.astype(np.float32)).to(t.bfloat16).view(t.int16).numpy().view(np.uint16)
    d = NbitsDev(p, c_dtype=c)
    uniform = zp == "f16_uniform"
    outs = {}
    try:
        for cand in (0, 1) + MX_CANDIDATES:
            Q.set_tuning(2, cand)
            outs[cand] = host_bits(d.run(uniform=uniform)).copy()
        Q.set_tuning(2, MX_CANDIDATES[0])
        for rep in range(2):  # repeated calls of the matrix-core form
            assert np.array_equal(host_bits(d.run(uniform=uniform)), outs[MX_CANDIDATES[0]])
        Q.set_tuning(2, MX_CANDIDATES[0])
        got = d.run(uniform=uniform)
    finally:
        Q.set_tuning(0, 0)
    for cand in (1,) + MX_CANDIDATES:
        assert np.array_equal(outs[cand], outs[0]), cand
    rows = sample_rows(N, 384, seed=902)
    ref = d.oracle(O, rows=rows)
    err = O.rel_l2(host_f64(got)[:, rows], ref)
    say(f"  relL2={err:.3e} over {len(rows)} columns (tol {TOL[c]:.0e})")
    assert err <= TOL[c]
    torch().cuda.synchronize()



def test_matrix_core_gemv_in_graph_replays():
    """The matrix-core form captured in a HIP graph: every replay (with eager work and
    synchronizations between them) gives the eager call's bits, and the same bits as the
    v_dot8 kernel."""
    t = torch()
    K, N = 5120, 16400
    assert Q.nbits_gemv_matrix_core_form(1, K, N, 2, 64)
    p = gen.nbits_problem(1, K, N, 2, 64, seed=905, zp="packed", bias=True)
    d = NbitsDev(p, c_dtype="f32")
    out = t.empty((1, N), dtype=t.float32, device="cuda")
    try:
        Q.set_tuning(2, 0)
        ref = host_bits(d.run()).copy()
        Q.set_tuning(2, MX_CANDIDATES[0])
        eager = host_bits(d.run()).copy()
        t.cuda.synchronize()
        cap = t.cuda.Stream()
        g = t.cuda.CUDAGraph()
        with t.cuda.stream(cap):
            with t.cuda.graph(g, stream=cap):
                d.run(out=out)
        t.cuda.synchronize()
        for rep in range(4):
            out.zero_()
            g.replay()
            t.cuda.synchronize()
            assert np.array_equal(host_bits(out), eager), rep
            d.run()  # eager work between replays
            t.cuda.synchronize()
    finally:
        Q.set_tuning(0, 0)
    assert np.array_equal(eager, ref)
