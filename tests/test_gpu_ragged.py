"""GPU parity of the ragged multi-token MoE matmul (qmoe_ragged_mm, Xfp16 x Wu4 -> Yfp16)
against the oracle, on bursts of T tokens with skewed top-k routing."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import inputs as gen
from gemm_qmm_nbits_amd import qmm as Q
from oracle import qmm_oracle as O

from gpu_util import TOL, assert_elementwise, dev, gamma, host_bits, host_f64, say, torch

pytestmark = pytest.mark.gpu


def skewed_ids(rng, T, E, k, skew=1.5):
    """Top-k experts of N(0,1) logits plus a popularity term -skew * log(1 + e): low
    experts are chosen far more often, the high ones rarely or never."""
    logits = rng.standard_normal((T, E)) - skew * np.log1p(np.arange(E))[None, :]
    return np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)


def burst(T, K, N, E, k, block, seed, zp, bias, skew=1.5):
    """A grouped burst: token rows gathered per (token, slot) in expert order."""
    rng = np.random.default_rng(seed)
    p = gen.qmoe_problem(1, K, N // 2, E, 1, block, seed=seed, zp=zp, bias=bias)  # fc1 is [E][N][..]
    fc = p["fc1"]
    ids = skewed_ids(rng, T, E, k, skew)
    order, offsets = O.group_by_expert(ids, E)
    X = gen.activations(rng, (T, K), "f16")
    Xg = X[order // k]
    return fc, ids, order, offsets, Xg


def check(fc, offsets, Xg, K, N, E, block, label):
    t = torch()
    fcd = {"W": dev(fc["W"]), "scales": dev(fc["scales"]),
           "zp": dev(fc["zp"]) if fc["zp"] is not None else None,
           "bias": dev(fc["bias"]) if fc["bias"] is not None else None}
    Xd = dev(Xg).view(t.float16)
    offs = dev(offsets.astype(np.int32))
    y = Q.qmoe_ragged_mm(Xd, offs, fcd, N, E, block)
    got = host_f64(y)
    mirr = O.qmoe_ragged_mm(Xg, offsets, fc, K, N, block, w_round="f16")
    exact = O.qmoe_ragged_mm(Xg, offsets, fc, K, N, block)
    err, raw = O.rel_l2(got, mirr), O.rel_l2(got, exact)
    say(f"  {label}: rows={Xg.shape[0]} relL2(mirrored)={err:.3e} relL2(exact)={raw:.3e}")
    assert err <= TOL["f16"] and raw <= TOL["f16"], (err, raw)
    # per-element bound of fp32 accumulation of the exact fp16 products
    x = O.f16_bits_to_f64(Xg)
    absdot = np.zeros_like(got)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            w = O._expert_dequant(fc, e, 4, K, block, N).astype(np.float64)
            absdot[r0:r1] = np.abs(x[r0:r1]) @ np.abs(O._round_operand(w, "f16")).T
    assert_elementwise(got, mirr, gamma(K + 2) * absdot, "f16", label)
    return y, host_bits(y).copy(), (Xd, offs, fcd)


@pytest.mark.parametrize("T", [16, 64, 256])
@pytest.mark.parametrize("block,zp,bias", [(32, True, True), (64, False, False), (128, True, False)])
def test_gpt_oss_fc1_bursts(T, block, zp, bias):
    """GPT-OSS-20B fc1 (32 experts, top-4, 2880 -> 5760), T-token bursts."""
    E, k, K, N = 32, 4, 2880, 5760
    fc, ids, order, offsets, Xg = burst(T, K, N, E, k, block, seed=1100 + T + block, zp=zp, bias=bias)
    check(fc, offsets, Xg, K, N, E, block, f"T={T} block={block}")


@pytest.mark.parametrize("T", [16, 64, 256])
@pytest.mark.parametrize("which", ["fc1", "fc2"])
def test_128_expert_bursts(T, which):
    """128 experts, top-8: fc1 2048 -> 1536 and fc2 768 -> 2048, zero points on."""
    E, k = 128, 8
    K, N = (2048, 1536) if which == "fc1" else (768, 2048)
    fc, ids, order, offsets, Xg = burst(T, K, N, E, k, 64, seed=1200 + T, zp=True, bias=False)
    assert (np.diff(offsets) == 0).any()    # the skew leaves some experts without rows
    check(fc, offsets, Xg, K, N, E, 64, f"{which} T={T}")


def test_ragged_edge_cases_and_repeats():
    """One expert holding every row (several 64-row tiles), a single row, empty experts in
    between, and repeated calls giving identical bits."""
    t = torch()
    E, K, N, block = 6, 1024, 300, 64
    rng = np.random.default_rng(1300)
    p = gen.qmoe_problem(1, K, N // 2, E, 1, block, seed=1300, zp=True, bias=True)
    fc = p["fc1"]
    for offsets in (np.array([0, 0, 0, 300, 300, 300, 300]), np.array([0, 1, 1, 1, 1, 1, 1]),
                    np.array([0, 17, 17, 80, 81, 81, 145])):
        R = int(offsets[-1])
        Xg = gen.activations(rng, (R, K), "f16")
        y, bits, args = check(fc, offsets, Xg, K, N, E, block, f"offsets={list(offsets)}")
        Xd, offs, fcd = args
        for _ in range(8):
            again = Q.qmoe_ragged_mm(Xd, offs, fcd, N, E, block)
            assert np.array_equal(host_bits(again), bits)
    t.cuda.synchronize()


def test_ragged_refusals():
    t = torch()
    X = t.zeros((4, 100), dtype=t.float16, device="cuda")   # K % 8 != 0
    offs = t.zeros(3, dtype=t.int32, device="cuda")
    w = {"W": t.zeros(16, dtype=t.uint8, device="cuda"), "scales": t.zeros(8, dtype=t.int16, device="cuda"),
         "zp": None, "bias": None}
    with pytest.raises(Q.QmmError) as e:
        Q.qmoe_ragged_mm(X, offs, w, 64, 2, 64)
    assert e.value.status == -5
    X2 = t.zeros((4, 128), dtype=t.float16, device="cuda")
    with pytest.raises(Q.QmmError) as e:
        Q.qmoe_ragged_mm(X2, offs, w, 64, 2, 16)
    assert e.value.status == -4
    with pytest.raises(Q.QmmError) as e:
        Q.qmoe_ragged_mm(X2, offs, w, 64, 2, 64, bits=2)
    assert e.value.status == -3
