"""The allocation-free MoE decode entry point (static device scratch) against the
allocating entry point, through the C ABI: bit-identical outputs on two calls in a row,
the second with a smaller input, in both activation modes."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import inputs as gen
from gemm_qmm_nbits_amd import qmm as Q

from gpu_util import dev, host_bits, say, torch

pytestmark = pytest.mark.gpu


def _dev_problem(p):
    t = torch()
    fc = {}
    for name in ("fc1", "fc2"):
        d = p[name]
        fc[name] = {"W": dev(d["W"]), "scales": dev(d["scales"]),
                    "zp": dev(d["zp"]) if d["zp"] is not None else None,
                    "bias": dev(d["bias"]) if d["bias"] is not None else None}
    return dev(p["X"]).view(t.float16), dev(p["ids"]), dev(p["rw"]), fc


@pytest.mark.parametrize("mode", [Q.QMOE_FP, Q.QMOE_INT8_ACT], ids=["fp", "int8"])
def test_noalloc_equals_allocating_entry(mode):
    t = torch()
    # two calls in a row on the same static scratch, the second smaller
    for T, H, I, E, k, block in ((4, 2048, 768, 128, 8, 64), (1, 1024, 512, 16, 4, 32)):
        say(f"noalloc mode={mode} T={T} H={H} I={I} E={E} k={k} block={block}")
        p = gen.qmoe_problem(T, H, I, E, k, block, seed=970 + T + mode, zp=True, bias=(T == 1))
        X, ids, rw, fc = _dev_problem(p)
        assert Q.qmoe_decode_scratch_bytes(T, H, I, k, mode) <= Q.QMOE_NOALLOC_SCRATCH_BYTES
        ref = Q.qmoe_decode_fused(X, ids, rw, fc["fc1"], fc["fc2"], H, I, E, block, mode=mode)
        out = t.full((T, H), float("nan"), dtype=t.float16, device="cuda")
        y = Q.qmoe_decode_fused_noalloc(X, ids, rw, fc["fc1"], fc["fc2"], H, I, E, block, out, mode=mode)
        t.cuda.synchronize()
        assert np.array_equal(host_bits(y), host_bits(ref))
        # and again on the scratch the call left behind
        y2 = Q.qmoe_decode_fused_noalloc(X, ids, rw, fc["fc1"], fc["fc2"], H, I, E, block, out, mode=mode)
        assert np.array_equal(host_bits(y2), host_bits(ref))


@pytest.mark.parametrize("mode", [Q.QMOE_FP, Q.QMOE_INT8_ACT], ids=["fp", "int8"])
def test_noalloc_single_launch_across_shapes(mode):
    """The single-launch form (forced) on the static scratch, alternating a larger and a
    smaller shape: every call finds its arrival count at zero (the sync words sit at the
    same place for every shape, never under another shape's h or codes) and matches the
    allocating entry."""
    t = torch()
    n1 = Q.num_candidates(Q.ENTRY_QMOE_FC1) * Q.num_candidates(Q.ENTRY_QMOE_FC2)
    shapes = ((4, 2048, 768, 128, 8, 64), (1, 1024, 512, 16, 4, 32))
    probs = []
    for T, H, I, E, k, block in shapes:
        p = gen.qmoe_problem(T, H, I, E, k, block, seed=980 + T + mode, zp=True, bias=True)
        probs.append(((T, H, I, E, k, block), _dev_problem(p)))
    Q.set_tuning(2, n1 + 1)   # single-launch candidate 1: fc2 streamed, one work-group per CU
    try:
        refs = []
        for (T, H, I, E, k, block), (X, ids, rw, fc) in probs:
            refs.append(host_bits(Q.qmoe_decode_fused(X, ids, rw, fc["fc1"], fc["fc2"], H, I, E, block,
                                                      mode=mode)).copy())
            assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == 1
        for rep in range(3):
            for i, ((T, H, I, E, k, block), (X, ids, rw, fc)) in enumerate(probs):
                say(f"noalloc single launch mode={mode} rep={rep} T={T} H={H}")
                out = t.full((T, H), float("nan"), dtype=t.float16, device="cuda")
                y = Q.qmoe_decode_fused_noalloc(X, ids, rw, fc["fc1"], fc["fc2"], H, I, E, block, out, mode=mode)
                assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == 1
                assert np.array_equal(host_bits(y), refs[i]), (rep, i)
    finally:
        Q.set_tuning(0, 0)


def test_noalloc_refuses_scratch_beyond_the_array():
    """A shape whose scratch exceeds the static array is refused before any launch."""
    t = torch()
    T, H, I, E, k = 512, 1024, 2048, 16, 8   # h alone needs 512 * 8 * 2048 * 2 bytes = 16 MiB
    assert Q.qmoe_decode_scratch_bytes(T, H, I, k, Q.QMOE_FP) > Q.QMOE_NOALLOC_SCRATCH_BYTES
    X = t.zeros((T, H), dtype=t.float16, device="cuda")
    ids = t.zeros((T, k), dtype=t.int32, device="cuda")
    rw = t.zeros((T, k), dtype=t.float32, device="cuda")
    w = t.zeros(16, dtype=t.uint8, device="cuda")
    s = t.zeros(16, dtype=t.int16, device="cuda")
    fc = {"W": w, "scales": s, "zp": None, "bias": None}
    out = t.empty((T, H), dtype=t.float16, device="cuda")
    with pytest.raises(Q.QmmError) as e:
        Q.qmoe_decode_fused_noalloc(X, ids, rw, fc, fc, H, I, E, 64, out)
    assert e.value.status == -7
