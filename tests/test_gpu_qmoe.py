"""GPU parity of the fused MoE decode (qmoe_decode_fused) against the oracle."""
import numpy as np
import pytest

from gemm_qmm_nbits_amd import inputs as gen
from gemm_qmm_nbits_amd import qmm as Q
from oracle import qmm_oracle as O

from gpu_util import TOL, dev, host_bits, host_f64, say, torch

pytestmark = pytest.mark.gpu


class MoeDev:
    def __init__(self, p):
        t = torch()
        self.p = p
        self.X = dev(p["X"]).view(t.float16)
        self.ids = dev(p["ids"])
        self.rw = dev(p["rw"])
        self.fc = {}
        for name in ("fc1", "fc2"):
            d = p[name]
            self.fc[name] = {"W": dev(d["W"]), "scales": dev(d["scales"]),
                             "zp": dev(d["zp"]) if d["zp"] is not None else None,
                             "bias": dev(d["bias"]) if d["bias"] is not None else None}

    def run(self, mode, X=None, ids=None, rw=None, out=None, scratch=None):
        p = self.p
        return Q.qmoe_decode_fused(self.X if X is None else X, self.ids if ids is None else ids,
                                   self.rw if rw is None else rw, self.fc["fc1"], self.fc["fc2"],
                                   p["H"], p["I"], p["E"], p["block"], mode=mode, out=out,
                                   scratch=scratch)

    def oracle(self, mode):
        p = self.p
        return O.qmoe_decode(p["X"], p["ids"], p["rw"], p["fc1"], p["fc2"], p["H"], p["I"],
                             p["block"], mode="int8" if mode == Q.QMOE_INT8_ACT else "fp")


def _check(d, mode, label):
    y = d.run(mode)
    ref = d.oracle(mode)
    err = O.rel_l2(host_f64(y), ref)
    say(f"  {label} relL2={err:.3e}")
    assert err <= TOL["f16"], (label, err)
    return y


MODES = [Q.QMOE_FP, Q.QMOE_INT8_ACT]


@pytest.mark.parametrize("mode", MODES, ids=["fp", "int8"])
@pytest.mark.parametrize("block", [32, 64, 128])
@pytest.mark.parametrize("zp,bias", [(False, False), (True, False), (False, True), (True, True)])
def test_gpt_oss_shape(mode, block, zp, bias):
    """GPT-OSS-20B-shaped layer: 32 experts, top-4, hidden = intermediate = 2880, one token."""
    c = gen.QMOE_GPT_OSS
    say(f"qmoe gpt-oss mode={mode} block={block} zp={zp} bias={bias}")
    p = gen.qmoe_problem(1, c["H"], c["I"], c["E"], c["k"], block,
                         seed=gen.config_seed(3, block + 2 * zp + bias), zp=zp, bias=bias)
    _check(MoeDev(p), mode, f"B={block} zp={zp} bias={bias}")


@pytest.mark.parametrize("mode", MODES, ids=["fp", "int8"])
@pytest.mark.parametrize("T", [1, 4, 8])
def test_128_experts_top8(mode, T):
    """128 experts, top-8, hidden 2048, intermediate 768, block 64, zero points, T tokens."""
    c = gen.QMOE_128
    say(f"qmoe 128/8 mode={mode} T={T}")
    p = gen.qmoe_problem(T, c["H"], c["I"], c["E"], c["k"], c["block"],
                         seed=gen.config_seed(4, T), zp=True, bias=False)
    _check(MoeDev(p), mode, f"T={T}")


@pytest.mark.parametrize("mode", MODES, ids=["fp", "int8"])
def test_batched_equals_single_calls(mode):
    """T tokens in one call give the bits of T separate single-token calls."""
    t = torch()
    p = gen.qmoe_problem(4, 1024, 512, 16, 4, 64, seed=901, zp=True, bias=True)
    d = MoeDev(p)
    yb = host_bits(d.run(mode)).copy()
    for i in range(4):
        yi = d.run(mode, X=d.X[i:i + 1].contiguous(), ids=d.ids[i:i + 1].contiguous(),
                   rw=d.rw[i:i + 1].contiguous())
        assert np.array_equal(host_bits(yi)[0], yb[i]), i
    t.cuda.synchronize()


def test_repeat_calls_bit_identical_int8():
    """129 calls of the int8-activation decode on one input give identical bits
    (a shape no other test uses, so the first call also runs the up-front timing)."""
    p = gen.qmoe_problem(1, 1408, 704, 24, 6, 32, seed=902, zp=True, bias=True)
    d = MoeDev(p)
    first = host_bits(d.run(Q.QMOE_INT8_ACT)).copy()
    out = torch().empty_like(d.X[:, :1408])
    for i in range(128):
        d.run(Q.QMOE_INT8_ACT, out=out)
        assert np.array_equal(host_bits(out), first), i
    assert O.rel_l2(first.view(np.float16).astype(np.float64), d.oracle(Q.QMOE_INT8_ACT)) <= TOL["f16"]


@pytest.mark.parametrize("mode", MODES, ids=["fp", "int8"])
def test_every_tiling_candidate_same_bits(mode):
    p = gen.qmoe_problem(2, 2880, 2880, 32, 4, 64, seed=903, zp=True, bias=True)
    d = MoeDev(p)
    n1 = Q.num_candidates(Q.ENTRY_QMOE_FC1)
    n2 = Q.num_candidates(Q.ENTRY_QMOE_FC2)
    outs = []
    try:
        for c in range(n1 * n2):
            Q.set_tuning(2, c)
            outs.append(host_bits(d.run(mode)).copy())
    finally:
        Q.set_tuning(0, 0)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_int8_activation_codes_bit_exact():
    """The int8 codes and scales of x and h the kernels use (kept in scratch) equal the
    oracle quantizer applied to x and to the kernels' own fp16 h."""
    t = torch()
    p = gen.qmoe_problem(2, 2048, 768, 16, 4, 64, seed=904, zp=True)
    d = MoeDev(p)
    T, H, I, k = 2, 2048, 768, 4
    nbytes = Q.qmoe_decode_scratch_bytes(T, H, I, k, Q.QMOE_INT8_ACT)
    scratch = t.zeros(nbytes, dtype=t.uint8, device="cuda")
    d.run(Q.QMOE_INT8_ACT, scratch=scratch)
    t.cuda.synchronize()
    raw = scratch.cpu().numpy()

    def a256(x):
        return (x + 255) // 256 * 256
    off_h = 33 * 256                 # after the sync words
    off_xq = off_h + a256(T * k * I * 2)
    off_xs = off_xq + a256(T * H)
    off_hq = off_xs + a256(T * (H // 32) * 4)
    off_hs = off_hq + a256(T * k * I)
    h = raw[off_h:off_h + T * k * I * 2].view(np.uint16).reshape(T, k, I)
    xq = raw[off_xq:off_xq + T * H].view(np.int8).reshape(T, H)
    xs = raw[off_xs:off_xs + T * (H // 32) * 4].view(np.float32).reshape(T, H // 32)
    hq = raw[off_hq:off_hq + T * k * I].view(np.int8).reshape(T, k, I)
    hs = raw[off_hs:off_hs + T * k * (I // 32) * 4].view(np.float32).reshape(T, k, I // 32)
    qx, sx = O.quantize_int8_groups(O.f16_bits_to_f64(p["X"]))
    assert np.array_equal(xq, qx) and np.array_equal(xs.view(np.uint32), sx.view(np.uint32))
    qh, sh = O.quantize_int8_groups(O.f16_bits_to_f64(h))
    assert np.array_equal(hq, qh) and np.array_equal(hs.view(np.uint32), sh.view(np.uint32))


def test_zero_tokens_and_refusals():
    t = torch()
    p = gen.qmoe_problem(1, 512, 256, 8, 2, 64, seed=905)
    d = MoeDev(p)
    # T = 0: nothing to do
    y = Q.qmoe_decode_fused(d.X[:0], d.ids[:0], d.rw[:0], d.fc["fc1"], d.fc["fc2"], 512, 256, 8, 64)
    assert y.shape == (0, 512)
    with pytest.raises(Q.QmmError) as e:
        Q.qmoe_decode_fused(d.X, d.ids, d.rw, d.fc["fc1"], d.fc["fc2"], 512, 256, 8, 16)
    assert e.value.status == -4
    with pytest.raises(Q.QmmError) as e:
        Q.qmoe_decode_fused(d.X, d.ids, d.rw, d.fc["fc1"], d.fc["fc2"], 512, 256, 8, 64, bits=2)
    assert e.value.status == -3
    small = t.empty(16, dtype=t.uint8, device="cuda")
    with pytest.raises(Q.QmmError) as e:
        Q.qmoe_decode_fused(d.X, d.ids, d.rw, d.fc["fc1"], d.fc["fc2"], 512, 256, 8, 64, scratch=small)
    assert e.value.status == -7


# ---- single-launch form (fp mode) --------------------------------------------------

def _fused_base():
    return Q.num_candidates(Q.ENTRY_QMOE_FC1) * Q.num_candidates(Q.ENTRY_QMOE_FC2)


SYNC_BYTES = 33 * 256   # slot 0 (top count, error flag) + 32 slots (sub-counter, phase)


def _sync_words(raw, T, H, I, k):
    """The sync words of the single-launch form (the first slots of the scratch layout)
    that must be zero after a call: slot 0 (top arrival count, error flag, unused words)
    and the 32 arrival sub-counters; the 32 phase copies must all be equal, 0 or 1."""
    w = raw[0:SYNC_BYTES].view(np.uint32)
    phases = w[65::64]
    assert phases.min() == phases.max() and phases[0] in (0, 1), phases
    return np.concatenate([w[:4], w[64::64]])


FUSED_CASES = [
    # (T, H, I, E, k, block, zp, bias)
    (1, 2880, 2880, 32, 4, 32, True, True),      # GPT-OSS-20B shape, 90 blocks per row
    (1, 2880, 2880, 32, 4, 128, False, True),    # ragged last block (22.5 blocks)
    (4, 2048, 768, 128, 8, 64, True, False),     # 128 experts, top-8, 4 tokens
    (3, 1000, 520, 10, 3, 64, True, True),       # ragged rows, tiles and blocks
]


FUSED_IDS = [f"T{c[0]}-H{c[1]}-I{c[2]}-B{c[5]}" for c in FUSED_CASES]


@pytest.mark.parametrize("mode", MODES, ids=["fp", "int8"])
@pytest.mark.parametrize("case", FUSED_CASES, ids=FUSED_IDS)
def test_single_launch_equals_two_kernel_forms(case, mode):
    """Every candidate of the single-launch form gives the bits of the two-kernel forms,
    leaves its arrival count at zero with no error (a wait that timed out would set one),
    and stays within the oracle tolerance.  A candidate whose LDS does not fit the shape
    falls back to the two-kernel form."""
    t = torch()
    T, H, I, E, k, block, zp, bias = case
    if mode == Q.QMOE_INT8_ACT and (H % 32 or I % 32):
        pytest.skip("int8 mode needs H and I multiples of 32")
    say(f"qmoe single launch mode={mode} T={T} H={H} I={I} E={E} k={k} block={block} zp={zp} bias={bias}")
    p = gen.qmoe_problem(T, H, I, E, k, block, seed=910 + T + block, zp=zp, bias=bias)
    d = MoeDev(p)
    base = _fused_base()
    nbytes = Q.qmoe_decode_scratch_bytes(T, H, I, k, mode)
    ran = []
    try:
        Q.set_tuning(2, 0)
        ref = host_bits(d.run(mode)).copy()
        assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == -1
        for c in range(Q.num_candidates(Q.ENTRY_QMOE_FUSED)):
            Q.set_tuning(2, base + c)
            scratch = t.zeros(nbytes, dtype=t.uint8, device="cuda")
            for rep in range(3):
                y = d.run(mode, scratch=scratch)
                assert np.array_equal(host_bits(y), ref), (c, rep)
                words = _sync_words(scratch.cpu().numpy(), T, H, I, k)
                assert not words.any(), (c, rep, np.nonzero(words)[0][:8])
            if Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == c:
                ran.append(c)
            else:
                assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == -1
    finally:
        Q.set_tuning(0, 0)
    say(f"  single-launch candidates run: {ran}")
    assert 0 in ran and 1 in ran  # one work-group per compute unit fits every case here
    err = O.rel_l2(ref.view(np.float16).astype(np.float64), d.oracle(mode))
    say(f"  relL2={err:.3e}")
    assert err <= TOL["f16"]


GRAPH_CASES = [(Q.QMOE_FP, 2, 2), (Q.QMOE_INT8_ACT, 2, 2), (Q.QMOE_INT8_ACT, 1, 1)]


@pytest.mark.parametrize("mode,cand,T", GRAPH_CASES,
                         ids=[f"{'fp' if m == Q.QMOE_FP else 'int8'}-c{c}-T{T}" for m, c, T in GRAPH_CASES])
def test_single_launch_graph_replays(mode, cand, T):
    """Calls of the single-launch form captured in a HIP graph and replayed several
    times, with eager calls on the same scratch between the replays, give the eager bits
    on every replay (its counters return to zero at the end of every launch)."""
    Q.set_tuning(2, _fused_base() + cand)
    try:
        _graph_replays(mode, cand, T)
    finally:
        Q.set_tuning(0, 0)


def _graph_replays(mode, cand, T):
    t = torch()
    H, I, E, k, block = 2880, 2880, 32, 4, 64
    p = gen.qmoe_problem(T, H, I, E, k, block, seed=921, zp=True, bias=True)
    d = MoeDev(p)
    rng = np.random.default_rng(922)
    routes = []
    for _ in range(3):
        ids, w = gen.routing(rng, T, E, k)
        routes.append((dev(ids), dev(w)))
    scratch = t.zeros(Q.qmoe_decode_scratch_bytes(T, H, I, k, mode), dtype=t.uint8, device="cuda")
    outs = [t.empty((T, H), dtype=t.float16, device="cuda") for _ in routes]
    eager = []
    for (ids, w), o in zip(routes, outs):
        eager.append(host_bits(d.run(mode, ids=ids, rw=w, out=o, scratch=scratch)).copy())
    assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == cand
    cap = t.cuda.Stream()
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(cap):
        with t.cuda.graph(g, stream=cap):
            for (ids, w), o in zip(routes, outs):
                d.run(mode, ids=ids, rw=w, out=o, scratch=scratch)
    t.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        t.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(host_bits(o), eager[i]), (rep, i)
        y = d.run(mode, ids=routes[rep % 3][0], rw=routes[rep % 3][1], scratch=scratch)
        assert np.array_equal(host_bits(y), eager[rep % 3]), rep
    assert not _sync_words(scratch.cpu().numpy(), T, H, I, k).any()


@pytest.mark.parametrize("form", ["tuned", "single-launch"])
def test_repeat_calls_bit_identical_fp(form):
    """129 calls of the fp decode on one input give identical bits: the form the
    up-front timing picks (a shape no other test uses, so the first call times), and
    the single-launch form forced."""
    p = gen.qmoe_problem(1, 1408, 704, 24, 6, 32, seed=923, zp=True, bias=True)
    d = MoeDev(p)
    if form == "single-launch":
        Q.set_tuning(2, _fused_base() + 1)
    try:
        first = host_bits(d.run(Q.QMOE_FP)).copy()
        if form == "single-launch":
            assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == 1
        out = torch().empty_like(d.X[:, :1408])
        for i in range(128):
            d.run(Q.QMOE_FP, out=out)
            assert np.array_equal(host_bits(out), first), i
    finally:
        Q.set_tuning(0, 0)
    assert O.rel_l2(first.view(np.float16).astype(np.float64), d.oracle(Q.QMOE_FP)) <= TOL["f16"]


@pytest.mark.parametrize("routing", ["shared", "one-expert"])
def test_experts_read_once_same_bits(routing):
    """The fc1 form that reads each expert's rows once for all its slots gives the bits of
    the per-slot forms: tokens that share all their experts, and every slot on one expert
    (repeated inside a token, so its 32 slots are split into units of 8)."""
    t = torch()
    T, H, I, E, k = 8, 1024, 512, 16, 4
    p = gen.qmoe_problem(T, H, I, E, k, 64, seed=930, zp=True, bias=True)
    if routing == "shared":
        p["ids"] = np.tile(np.array([[3, 9, 0, 14]], dtype=np.int32), (T, 1))
    else:
        p["ids"] = np.full((T, k), 5, dtype=np.int32)
    d = MoeDev(p)
    n1 = Q.num_candidates(Q.ENTRY_QMOE_FC1)
    once = n1 - 1          # fc1 candidate: experts read once (the last one)
    per_slot = 2           # per-slot form, one row per lane
    outs = []
    try:
        for fc1, fc2 in ((per_slot, per_slot), (once, 0), (once, per_slot)):
            Q.set_tuning(2, fc1 + n1 * fc2)
            outs.append(host_bits(d.run(Q.QMOE_FP)).copy())
    finally:
        Q.set_tuning(0, 0)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    err = O.rel_l2(outs[0].view(np.float16).astype(np.float64), d.oracle(Q.QMOE_FP))
    say(f"  {routing} relL2={err:.3e}")
    assert err <= TOL["f16"]
    t.cuda.synchronize()


# ---- error state, capture and the wait's status ---------------------------------------

@pytest.mark.parametrize("mode", MODES, ids=["fp", "int8"])
def test_first_call_over_pending_error(mode):
    """The first call of a shape no other test uses, made while an unrelated HIP error is
    pending, succeeds and is within tolerance: the error state is cleared on entry, so
    neither the up-front timing nor the call reports it."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime already loaded by torch
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    t = torch()
    p = gen.qmoe_problem(1, 1536, 512, 12, 3, 64, seed=940 + mode, zp=True, bias=True)
    d = MoeDev(p)
    # output and scratch come first: torch checks the error state after its own launches
    out = t.empty((1, 1536), dtype=t.float16, device="cuda")
    scratch = t.zeros(Q.qmoe_decode_scratch_bytes(1, 1536, 512, 3, mode), dtype=t.uint8, device="cuda")
    t.cuda.synchronize()
    # hipSetDevice on an invalid ordinal records hipErrorInvalidDevice without touching the GPU
    assert hip.hipSetDevice(9999) != 0
    y = d.run(mode, out=out, scratch=scratch)
    err = O.rel_l2(host_f64(y), d.oracle(mode))
    say(f"  pending error mode={mode} relL2={err:.3e}")
    assert err <= TOL["f16"], err


@pytest.mark.parametrize("mode", MODES, ids=["fp", "int8"])
def test_first_call_under_capture(mode):
    """The first call of an untimed shape inside a stream capture: nothing is timed (the
    timing's synchronization would break the capture), and every replay, with eager calls
    in between, gives the bits of the later timed eager call."""
    t = torch()
    T, H, I, E, k = 2, 1280, 640, 20, 4
    p = gen.qmoe_problem(T, H, I, E, k, 64, seed=950 + mode, zp=True, bias=False)
    d = MoeDev(p)
    scratch = t.zeros(Q.qmoe_decode_scratch_bytes(T, H, I, k, mode), dtype=t.uint8, device="cuda")
    out = t.empty((T, H), dtype=t.float16, device="cuda")
    t.cuda.synchronize()
    cap = t.cuda.Stream()
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(cap):
        with t.cuda.graph(g, stream=cap):
            d.run(mode, out=out, scratch=scratch)
    t.cuda.synchronize()
    eager = host_bits(d.run(mode, scratch=scratch)).copy()   # first uncaptured call: times
    for rep in range(3):
        out.zero_()
        g.replay()
        t.cuda.synchronize()
        assert np.array_equal(host_bits(out), eager), rep
        assert np.array_equal(host_bits(d.run(mode, scratch=scratch)), eager), rep
    err = O.rel_l2(eager.view(np.float16).astype(np.float64), d.oracle(mode))
    assert err <= TOL["f16"], err
    assert not Q.qmoe_decode_status(scratch, T, H, I, k, mode)


@pytest.mark.parametrize("mode", MODES, ids=["fp", "int8"])
def test_untimed_default_is_single_launch(mode):
    """With tuning off nothing is timed and the decode runs as one launch (the
    single-launch candidate with fc2 streamed, one work-group per CU) where its plan
    fits; its bits equal the two-kernel form's."""
    T, H, I, E, k = 1, 2880, 2880, 32, 4
    p = gen.qmoe_problem(T, H, I, E, k, 64, seed=965 + mode, zp=True, bias=True)
    d = MoeDev(p)
    try:
        Q.set_tuning(1, 0)
        one = host_bits(d.run(mode)).copy()
        assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == 1
        Q.set_tuning(2, 0)  # the two-kernel form
        two = host_bits(d.run(mode)).copy()
        assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == -1
    finally:
        Q.set_tuning(0, 0)
    assert np.array_equal(one, two)


def test_decode_status_clear_after_single_launch_calls():
    """qmoe_decode_status reports no wait that gave up after calls of the single-launch
    form, and refuses a scratch buffer smaller than the layout."""
    t = torch()
    T, H, I, E, k = 1, 2880, 2880, 32, 4
    p = gen.qmoe_problem(T, H, I, E, k, 64, seed=960, zp=False, bias=False)
    d = MoeDev(p)
    scratch = t.zeros(Q.qmoe_decode_scratch_bytes(T, H, I, k, Q.QMOE_FP), dtype=t.uint8, device="cuda")
    Q.set_tuning(2, _fused_base() + 0)
    try:
        for _ in range(5):
            y = d.run(Q.QMOE_FP, scratch=scratch)
        assert Q.tuned_choice(Q.ENTRY_QMOE_FUSED) == 0
    finally:
        Q.set_tuning(0, 0)
    assert np.all(np.isfinite(host_f64(y)))
    assert Q.qmoe_decode_status(scratch, T, H, I, k, Q.QMOE_FP) is False
    with pytest.raises(Q.QmmError) as e:
        Q.qmoe_decode_status(scratch[:64], T, H, I, k, Q.QMOE_FP)
    assert e.value.status == -7
