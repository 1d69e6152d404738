"""Benchmark of the fused low-bit dequantize-matmul path on one MI355X.

One step = one decode pass (M = 1) over the four phi4-14B-shaped 2-bit
MatMulNBits layers (qkv 5120x7680, gate_up 5120x35840, down 17920x5120,
lm_head 5120x100352; block 64, fp16 scales, uniform zero point 1.5, fp32 A and
C).  Weights are resident in HBM; every layer has its own pool of copies of at
least 1 GiB (four times the 256 MB last-level cache), so every step reads them
cold.  `value` is the weight bytes streamed per step divided by the step time
(HIP graphs of eight consecutive steps, each on its own weight copies, replayed
back to back; one-step graphs are timed too and reported beside it).

Extra legs in the same JSON line: per-layer kernel times (one HIP event pair per
launch), the tiny u4 GEMV, the 40-layer phi4 stack, the prefill matmul at
M = 2048, the codebook matmul (plain and nested absmax), 3/4/8-bit weights, the
fused MoE decode (GPT-OSS-20B shape at blocks 32/64/128 in both activation modes,
and the 128-expert top-8 shape, fresh routing per call), the ragged MoE matmul,
the device Q/DQ ops, ceilings (a 128-bit streaming read, a copy, hipBLASLt fp16)
and an N sweep.  All timing is on the stream the kernels are launched on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--legs ...]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2516.6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="decode,tiny,stack,prefill,qmoe,codebook,wide,ragged,qdq,ceilings,nsweep",
                    help="comma list of decode,tiny,stack,prefill,qmoe,codebook,wide,ragged,qdq,ceilings,"
                         "nsweep (the GEMV at N around the gate_up and lm_head widths); copycal: a plain "
                         "copy for counter calibration")
    ap.add_argument("--decode-shapes", default="qkv,gate_up,down,lm_head",
                    help="subset of the phi4 layers in the decode step (profiling runs)")
    return ap.parse_args()


def to_dev(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda()
    return torch.from_numpy(x).cuda()


def weight_bytes_nbits(K, N, bits=2, block=64):
    nblk = (K + block - 1) // block
    return N * nblk * block * bits // 8 + N * nblk * 2   # packed codes + fp16 scales


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

class Timer:
    """Timing on the current stream.

    graph_us: a captured HIP graph of launches, replayed in bursts back to back; the
    median over bursts of the mean time per launch (so it includes the gap between
    dependent launches).
    kernel_us: the execution time of each kernel the library launches, from a pair of
    HIP events that the launch itself records (hipExtLaunchKernel, the library's launch
    timing); the stream is first held busy by streaming reads so that the launches run
    back to back.  Per call: the sum over the call's launches; the mean over calls.
    event_us: one event pair recorded around each call (torch kernels), behind the same hold.
    """

    def __init__(self):
        import torch
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self._hold = None

    def capture(self, fns):
        torch = self.torch
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for fn in fns:
                    fn()
        torch.cuda.synchronize()
        return g

    def graph_us(self, g, per_replay, bursts=9):
        torch = self.torch
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(bursts + 1)]
        ev[0].record(self.stream)
        for b in range(bursts):
            g.replay()
            ev[b + 1].record(self.stream)
        torch.cuda.synchronize()
        per = sorted(ev[b].elapsed_time(ev[b + 1]) * 1e3 / per_replay for b in range(bursts))
        return per[bursts // 2]

    def hold(self, n=24):
        """Keep the stream busy for a few ms with streaming reads of 1 GiB."""
        torch = self.torch
        from gemm_qmm_nbits_amd import qmm as Q
        if self._hold is None:
            self._hold = (torch.empty(1 << 30, dtype=torch.uint8, device="cuda"),
                          torch.empty(4096, dtype=torch.int32, device="cuda"))
        buf, sink = self._hold
        for _ in range(n):
            Q.hbm_read_probe(buf, sink, 4096, stream=self.stream)

    def kernel_us(self, fns):
        """Kernel execution time per call of fns (library calls), from launch timing."""
        from gemm_qmm_nbits_amd import qmm as Q
        torch = self.torch
        for fn in fns:
            fn()
        torch.cuda.synchronize()
        n = len(fns)
        self.hold(8 + n // 2)
        Q.launch_timing_begin(16 * n)
        try:
            for fn in fns:
                fn()
        finally:
            us = Q.launch_timing_end(16 * n)
        if not us or len(us) % n:
            raise RuntimeError(f"launch timing: {len(us)} launches over {n} calls")
        per = len(us) // n
        calls = [sum(us[i * per:(i + 1) * per]) for i in range(n)]
        return {"kernel_us": float(np.mean(calls)), "kernel_us_median": float(np.median(calls)),
                "launches_per_call": per}

    def event_us(self, fns):
        """Mean time of fns from one event pair around each call, behind a hold."""
        torch = self.torch
        for fn in fns:
            fn()
        torch.cuda.synchronize()
        n = len(fns)
        s = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.hold(8 + n // 2)
        for i, fn in enumerate(fns):
            s[i].record(self.stream)
            fn()
            e[i].record(self.stream)
        torch.cuda.synchronize()
        return {"event_us": float(np.mean([s[i].elapsed_time(e[i]) * 1e3 for i in range(n)]))}

    def release(self):
        self._hold = None


def pool_copies(nbytes, floor=2):
    """Copies of a weight set whose total reaches 1 GiB (4x the 256 MB last-level cache)."""
    return max(floor, int(np.ceil((1 << 30) / nbytes)) + 1)


def nbits_copies(K, N, bits, count, seed, first=None):
    """`count` device copies of (W, scales) for a [N, K] layer, block 64: copy 0 from
    `first` (seeded numpy arrays) when given, the rest random bytes and fp16 scales in
    [0.01, 0.05] from a seeded device generator."""
    import torch
    nblk = (K + 63) // 64
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for c in range(count):
        if c == 0 and first is not None:
            out.append((to_dev(first[0]), to_dev(first[1])))
            continue
        W = torch.randint(0, 256, (N, nblk * 8 * bits), dtype=torch.uint8, device="cuda", generator=g)
        S = (torch.rand((N, nblk), device="cuda", generator=g) * 0.04 + 0.01).half()
        out.append((W, S))
    return out


# ---------------------------------------------------------------------------
# decode leg: phi4 2-bit M = 1
# ---------------------------------------------------------------------------

def decode_leg(args, T):
    """Decode step = the four phi4 layers at M = 1.  Each layer has its own pool of weight
    copies of >= 1 GiB; step i uses copy i mod (pool size) of every layer, and the steps
    are captured as HIP graphs and replayed back to back (host launch gaps excluded)."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q

    want = args.decode_shapes.split(",")
    shapes = [(n, kn) for n, kn in gen.PHI4_SHAPES.items() if n in want]
    step_bytes = sum(weight_bytes_nbits(K, N) for _, (K, N) in shapes)
    layers = []
    for name, (K, N) in shapes:
        si = list(gen.PHI4_SHAPES).index(name)
        p = gen.nbits_problem(1, K, N, 2, 64, seed=gen.config_seed(1, si), zp="none", scale_range=(0.01, 0.05))
        copies = pool_copies(weight_bytes_nbits(K, N))
        layers.append({"name": name, "K": K, "N": N, "A": to_dev(p["A"]),
                       "C": torch.empty((1, N), dtype=torch.float32, device="cuda"),
                       "pool": nbits_copies(K, N, 2, copies, 5000 + si, first=(p["W"], p["scales"]))})
        del p
    log(f"[decode] {len(shapes)} shapes, {step_bytes / 1e6:.1f} MB weights/step, copies "
        + ",".join(str(len(L["pool"])) for L in layers))

    def launch(L, c):
        W, S = L["pool"][c % len(L["pool"])]
        Q.qmm_nbits(L["A"], W, S, L["K"], 2, 64, None, Q.QMM_ZP_UNIFORM, 1.5, out=L["C"])

    for L in layers:       # eager warm-up: the first call of each shape takes the tiling choice
        for c in range(len(L["pool"])):
            launch(L, c)
    torch.cuda.synchronize()
    eager_ref = []
    for L in layers:
        launch(L, 0)
        torch.cuda.synchronize()
        eager_ref.append(L["C"].clone())
    period = max(len(L["pool"]) for L in layers)
    step_graphs = [T.capture([lambda L=L, i=i: launch(L, i) for L in layers]) for i in range(period)]
    # The timed steps run as graphs of GROUP consecutive steps, each step on its own
    # weight copies: in a serving loop a decode step sits inside a larger captured graph
    # (as in the stack leg), and a graph of only four launches adds a graph boundary per
    # step.  The one-step graphs are timed too and reported beside it.
    GROUP = 8
    ngroups = (period + GROUP - 1) // GROUP
    group_graphs = [T.capture([lambda L=L, i=(j * GROUP + t) % period: launch(L, i)
                               for t in range(GROUP) for L in layers]) for j in range(ngroups)]
    for i in range(args.warmup):
        step_graphs[i % period].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    nfull, rem = divmod(args.steps, GROUP)
    t0 = time.perf_counter()
    e0.record(T.stream)
    for j in range(nfull):
        group_graphs[j % ngroups].replay()
    for i in range(rem):
        step_graphs[(nfull * GROUP + i) % period].replay()
    e1.record(T.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    # the same steps, one graph per step
    e0.record(T.stream)
    for i in range(args.steps):
        step_graphs[i % period].replay()
    e1.record(T.stream)
    torch.cuda.synchronize()
    step_ms_one = e0.elapsed_time(e1) / args.steps
    # the graph replays give the eager outputs
    for L in layers:
        L["C"].zero_()
    step_graphs[0].replay()
    torch.cuda.synchronize()
    same = all(torch.equal(r, L["C"]) for r, L in zip(eager_ref, layers))
    del step_graphs, group_graphs
    shapes_out = {}
    for L in layers:
        K, N, c = L["K"], L["N"], len(L["pool"])
        b = weight_bytes_nbits(K, N)
        n = max(c, 20)
        g = T.capture([lambda i=i: launch(L, i) for i in range(n)])
        gus = T.graph_us(g, n)
        del g
        ku = T.kernel_us([lambda i=i: launch(L, i) for i in range(2 * c if c < 20 else c)])
        ev = T.event_us([lambda i=i: launch(L, i) for i in range(2 * c if c < 20 else c)])
        hot = T.kernel_us([lambda: launch(L, 0) for _ in range(20)])
        shapes_out[L["name"]] = {
            "K": K, "N": N, "weight_MB": round(b / 1e6, 3), "copies": c,
            "graph_us": round(gus, 2), "GBps_graph": round(b / gus / 1e3, 1),
            "kernel_us": round(ku["kernel_us"], 2), "GBps": round(b / ku["kernel_us"] / 1e3, 1),
            "frac_hbm": round(b / ku["kernel_us"] / 1e3 / HBM_PEAK_GBS, 4),
            "event_pair_us": round(ev["event_us"], 2),
            "hot_kernel_us": round(hot["kernel_us"], 2),
            "hot_GBps": round(b / hot["kernel_us"] / 1e3, 1)}
    del layers
    torch.cuda.empty_cache()
    return {"step_bytes": step_bytes, "step_ms": step_ms, "step_ms_one_step_graphs": step_ms_one,
            "steps_per_graph": GROUP, "wall_s": wall, "shapes": shapes_out,
            "graph_replay_matches_eager": bool(same)}


def tiny_leg(T):
    """The tiny u4 GEMV (M = 1, K = 256, N = 128, block 64, packed zero point 8, fp32):
    a launch-latency case, reported in us."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q
    p = gen.nbits_problem(1, 256, 128, 4, 64, seed=gen.config_seed(0), zp="packed8")
    A, W, S, Z = to_dev(p["A"]), to_dev(p["W"]), to_dev(p["scales"]), to_dev(p["zp"])
    C = torch.empty((1, 128), dtype=torch.float32, device="cuda")

    def call():
        Q.qmm_nbits(A, W, S, 256, 4, 64, Z, Q.QMM_ZP_PACKED, 0.0, out=C)

    g = T.capture([call] * 20)
    gus = T.graph_us(g, 20)
    ku = T.kernel_us([call] * 20)
    return {"M": 1, "K": 256, "N": 128, "bits": 4, "graph_us": round(gus, 2),
            "kernel_us": round(ku["kernel_us"], 2), "launches": ku["launches_per_call"]}


# ---------------------------------------------------------------------------
# stack leg: the phi4-14B 2-bit decode stack, 40 x (qkv, gate_up, down) + lm_head
# ---------------------------------------------------------------------------

def stack_leg(args, layers=40, reps=10):
    """One decode token through 40 layers of distinct phi4 2-bit weights (qkv, gate_up,
    down) and the lm_head, M = 1, fp32 A/C, uniform zp 1.5, captured as one HIP graph
    of 121 GEMV launches (3.68 GB of weights: every replay streams them cold)."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q

    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    shapes = [gen.PHI4_SHAPES[n] for n in ("qkv", "gate_up", "down")]
    calls = []
    total = 0
    for li in range(layers + 1):
        for (K, N) in (shapes if li < layers else [gen.PHI4_SHAPES["lm_head"]]):
            nblk = (K + 63) // 64
            W = torch.randint(0, 256, (N, nblk * 16), dtype=torch.uint8, device="cuda", generator=g)
            S = (torch.rand((N, nblk), device="cuda", generator=g) * 0.04 + 0.01).half()
            A = torch.randn((1, K), device="cuda", generator=g)
            C = torch.empty((1, N), device="cuda")
            calls.append((A, W, S, K, C))
            total += weight_bytes_nbits(K, N)

    def token():
        for (A, W, S, K, C) in calls:
            Q.qmm_nbits(A, W, S, K, 2, 64, None, Q.QMM_ZP_UNIFORM, 1.5, out=C)

    token()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap):
            token()
    torch.cuda.synchronize()
    gr.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        gr.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = total / (ms * 1e-3) / 1e9
    del gr, calls
    torch.cuda.empty_cache()
    log(f"[stack] {layers} layers + lm_head: {ms:.3f} ms/token")
    return {"layers": layers, "weight_GB_per_token": round(total / 1e9, 3), "ms_per_token": round(ms, 4),
            "tok_per_s": round(1e3 / ms, 1), "weight_GBps": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "launches_per_token": 3 * layers + 1}


# ---------------------------------------------------------------------------
# codebook leg: 16-entry codebook 4-bit weights, M in {1, 4, 16, 64}, bf16 A/C
# ---------------------------------------------------------------------------

def codebook_leg(T):
    """Weight GB/s of qmm_codebook4 at the four codebook shapes for M = 1, 4, 16, 64:
    bf16 A and C, block 64, weight copies >= 1 GiB per shape (M = 1, and M = 4 on at
    most 2^24 codes: weight-streaming GEMV; otherwise matrix cores).  Also the nested-absmax form (uint8 absmax codes through
    a 256-entry table and per-256-block scales) at M = 1."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q

    out = {}
    for si, (name, (K, N)) in enumerate(gen.CODEBOOK_SHAPES.items()):
        nblk = (K + 63) // 64
        wbytes = N * nblk * (32 + 4)  # packed codes + fp32 absmax
        copies = pool_copies(wbytes)
        base = gen.codebook_problem(1, K, N, seed=gen.config_seed(2, 1000 + si))
        cb = to_dev(base["codebook"])
        g = torch.Generator(device="cuda")
        g.manual_seed(N + si)
        Ws = [torch.randint(0, 256, (N, nblk * 32), dtype=torch.uint8, device="cuda", generator=g)
              for _ in range(copies)]
        ams = [(torch.rand((N, nblk), device="cuda", generator=g) * 0.09 + 0.01) for _ in range(copies)]
        for M in gen.CODEBOOK_M:
            A = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
            C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            wsb = Q.lib().qmm_codebook4_workspace_bytes(M, K, N, Q.QMM_BF16)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

            def call(i, A=A, C=C, ws=ws, wsb=wsb):
                Q.qmm_codebook4(A, Ws[i % copies], ams[i % copies], cb, K, 64, None, out=C,
                                workspace=ws if wsb else None)

            n = max(copies, 20)
            gr = T.capture([lambda i=i: call(i) for i in range(n)])
            gus = T.graph_us(gr, n)
            del gr
            ku = T.kernel_us([lambda i=i: call(i) for i in range(n)])
            out[f"{name} M={M}"] = {
                "K": K, "N": N, "M": M, "graph_us": round(gus, 2), "kernel_us": round(ku["kernel_us"], 2),
                "weight_GBps": round(wbytes / ku["kernel_us"] / 1e3, 1),
                "frac_hbm": round(wbytes / ku["kernel_us"] / 1e3 / HBM_PEAK_GBS, 4),
                "path": "gemv" if M < 4 or (M == 4 and N * K <= 1 << 24) else "matrix cores"}
        # nested absmax at M = 1: codes 1 B per block + table + scales per 256 blocks
        nbytes = N * nblk * (32 + 1) + 256 * 4 + ((N * nblk + 255) // 256) * 4
        na = gen.nested_absmax_inputs(np.random.default_rng(900 + si), N, nblk)
        table, nscales = to_dev(na["table"]), to_dev(na["scales"])
        nas = [{"codes": to_dev(na["codes"]) if c == 0 else
                torch.randint(0, 256, (N, nblk), dtype=torch.uint8, device="cuda", generator=g),
                "table": table, "scales": nscales, "offset": float(na["offset"]), "group": na["group"]}
               for c in range(copies)]
        A = torch.randn((1, K), device="cuda", generator=g).to(torch.bfloat16)
        C = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
        wsb = Q.lib().qmm_codebook4_nested_workspace_bytes(1, K, N, Q.QMM_BF16, 64)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

        def ncall(i):
            Q.qmm_codebook4_nested(A, Ws[i % copies], nas[i % copies], cb, K, 64, None, out=C, workspace=ws)

        n = max(copies, 20)
        gr = T.capture([lambda i=i: ncall(i) for i in range(n)])
        gus = T.graph_us(gr, n)
        del gr
        out[f"{name} M=1 nested absmax"] = {"K": K, "N": N, "M": 1, "graph_us": round(gus, 2),
                                            "weight_GBps_graph": round(nbytes / gus / 1e3, 1),
                                            "note": "absmax decode launch + GEMV per call"}
        del Ws, ams, nas
        torch.cuda.empty_cache()
    log(f"[codebook] {len(out)} cases")
    return out


# ---------------------------------------------------------------------------
# prefill leg: phi4 2-bit M = 2048 on the matrix cores
# ---------------------------------------------------------------------------

def prefill_leg(args, M=2048, calls=5):
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q

    out = {}
    tot_flop = 0.0
    tot_ms = 0.0
    for si, (name, (K, N)) in enumerate(gen.PHI4_SHAPES.items()):
        p = gen.nbits_problem(1, K, N, 2, 64, seed=gen.config_seed(1, 20 + si), zp="none",
                              scale_range=(0.01, 0.05))
        W, S = to_dev(p["W"]), to_dev(p["scales"])
        A = torch.randn((M, K), dtype=torch.float32, device="cuda",
                        generator=torch.Generator(device="cuda").manual_seed(si))
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(Q.lib().qmm_nbits_workspace_bytes(M, K, N, Q.QMM_F32), dtype=torch.uint8,
                         device="cuda")
        stream = torch.cuda.current_stream()
        for _ in range(2):
            Q.qmm_nbits(A, W, S, K, 2, 64, None, Q.QMM_ZP_UNIFORM, 1.5, out=C, workspace=ws,
                        stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            Q.qmm_nbits(A, W, S, K, 2, 64, None, Q.QMM_ZP_UNIFORM, 1.5, out=C, workspace=ws,
                        stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / calls
        flop = 2.0 * M * N * K
        tot_flop += flop
        tot_ms += ms
        out[name] = {"K": K, "N": N, "M": M, "us": round(ms * 1e3, 1),
                     "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 1),
                     "frac_mfma_f16": round(flop / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
        del A, C, ws, W, S
        torch.cuda.empty_cache()
    tf = tot_flop / (tot_ms * 1e-3) / 1e12
    return {"shapes": out, "TFLOPs": round(tf, 1), "frac_mfma_f16": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "note": "cast of fp32 A to fp16 included in each call"}


# ---------------------------------------------------------------------------
# MoE decode leg
# ---------------------------------------------------------------------------

def qmoe_bytes(H, I, block, zp, bias, n_experts):
    def per(nout, kin):
        nblk = (kin + block - 1) // block
        b = nout * nblk * block // 2 + nout * nblk * 2
        if zp:
            b += nout * ((nblk + 1) // 2)
        if bias:
            b += nout * 2
        return b
    return n_experts * (per(2 * I, H) + per(H, I))


def qmoe_layer(T_, H, I, E, k, block, zp, bias):
    """Device copies (>= 1 GiB together) of one MoE layer's fc1/fc2 weights, and X."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    layer_bytes = qmoe_bytes(H, I, block, zp, bias, E)
    copies = max(3, int(np.ceil((1 << 30) / layer_bytes)))
    p = gen.qmoe_problem(T_, H, I, E, k, block, seed=gen.config_seed(3 if E == 32 else 4, T_ + block),
                         zp=zp, bias=bias)
    first = {}
    for fc in ("fc1", "fc2"):
        src = p[fc]
        first[fc] = {"W": to_dev(src["W"]), "scales": to_dev(src["scales"]),
                     "zp": to_dev(src["zp"]) if src["zp"] is not None else None,
                     "bias": to_dev(src["bias"]) if src["bias"] is not None else None}
    fcs = [first] + [{fc: {key: (None if v is None else v.clone()) for key, v in first[fc].items()}
                      for fc in ("fc1", "fc2")} for _ in range(copies - 1)]
    return {"fcs": fcs, "X": to_dev(p["X"]).view(torch.float16), "copies": copies}


def qmoe_leg(T, name, layer, T_, H, I, E, k, block, zp, bias, mode, calls=48):
    """Fused MoE decode: `calls` calls with fresh routing each over whole-layer weight
    copies (>= 1 GiB), captured in one HIP graph and replayed; mean per call (tok/s).  Also
    the kernel execution time per call (the sum over its launches, from launch timing),
    which the weight GB/s uses."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q

    fcs, X, copies = layer["fcs"], layer["X"][:T_], layer["copies"]
    assert X.shape[0] == T_
    rng = np.random.default_rng(7 + block)
    routes = []
    n_unique = []
    for i in range(calls):
        ids, w = gen.routing(rng, T_, E, k)
        routes.append((to_dev(ids), to_dev(w)))
        n_unique.append(len(np.unique(ids)))
    Y = torch.empty((T_, H), dtype=torch.float16, device="cuda")
    scratch = torch.zeros(Q.qmoe_decode_scratch_bytes(T_, H, I, k, mode), dtype=torch.uint8, device="cuda")

    def call(i):
        d = fcs[i % copies]
        Q.qmoe_decode_fused(X, routes[i][0], routes[i][1], d["fc1"], d["fc2"], H, I, E, block,
                            mode=mode, out=Y, scratch=scratch)

    for i in range(min(calls, 4)):   # eager: the first call times the tiling candidates
        call(i)
    torch.cuda.synchronize()
    g = T.capture([lambda i=i: call(i) for i in range(calls)])
    us = T.graph_us(g, calls, bursts=5)
    del g
    ku = T.kernel_us([lambda i=i: call(i) for i in range(calls)])
    gave_up = Q.qmoe_decode_status(scratch, T_, H, I, k, mode)
    uniq = float(np.mean(n_unique))
    per_expert = qmoe_bytes(H, I, block, zp, bias, 1)
    kus = ku["kernel_us"]
    return {"name": name, "T": T_, "H": H, "I": I, "E": E, "k": k, "block": block, "zp": zp,
            "bias": bias, "mode": "int8" if mode == Q.QMOE_INT8_ACT else "fp",
            "us_per_call": round(us, 2), "tok_per_s": round(T_ / (us * 1e-6), 1), "kernel_us": round(kus, 2),
            "weight_MB_per_call": round(uniq * per_expert / 1e6, 2),
            "weight_GBps": round(uniq * per_expert / kus / 1e3, 1),
            "frac_hbm": round(uniq * per_expert / kus / 1e3 / HBM_PEAK_GBS, 4),
            "unique_experts_mean": uniq, "launches_per_call": ku["launches_per_call"],
            "wait_gave_up": bool(gave_up)}


def qmoe_legs(T):
    from gemm_qmm_nbits_amd import qmm as Q
    import torch
    out = []
    for block, zp, bias in ((32, False, False), (64, False, False), (128, False, False), (32, True, True)):
        layer = qmoe_layer(1, 2880, 2880, 32, 4, block, zp, bias)
        for mode in (Q.QMOE_FP, Q.QMOE_INT8_ACT):
            out.append(qmoe_leg(T, "gpt-oss-20b", layer, 1, 2880, 2880, 32, 4, block, zp, bias, mode))
        del layer
        torch.cuda.empty_cache()
    layer = qmoe_layer(8, 2048, 768, 128, 8, 64, True, False)
    for T_ in (1, 4, 8):
        out.append(qmoe_leg(T, "128x768 top-8", layer, T_, 2048, 768, 128, 8, 64, True, False, Q.QMOE_FP))
    del layer
    torch.cuda.empty_cache()
    log(f"[qmoe] {len(out)} cases")
    return out


def ragged_leg(T):
    """Ragged multi-token MoE matmul at the GPT-OSS fc1 shape (E = 32, K = 2880, N = 5760,
    block 64, no zero point) on bursts of T tokens x top-4, rows grouped by expert:
    TFLOP/s and the weight bytes of the experts the burst touches."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q
    E, k, K, N, block = 32, 4, 2880, 5760, 64
    p = gen.qmoe_problem(1, K, N // 2, E, 1, block, seed=gen.config_seed(3, 777))
    fc = p["fc1"]
    w0 = {"W": to_dev(fc["W"]), "scales": to_dev(fc["scales"]), "zp": None, "bias": None}
    ws = [w0] + [{"W": w0["W"].clone(), "scales": w0["scales"].clone(), "zp": None, "bias": None}
                 for _ in range(3)]     # 4 copies of 276 MB: every call reads its experts cold
    per_expert = N * ((K + block - 1) // block) * (block // 2 + 2)
    rng = np.random.default_rng(31)
    res = []
    for T_ in (16, 64, 256, 1024):
        ids, _ = gen.routing(rng, T_, E, k)
        counts = np.bincount(ids.ravel(), minlength=E)
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        R = T_ * k
        X = torch.randn((R, K), device="cuda").half()
        offs = to_dev(offsets)
        Y = torch.empty((R, N), dtype=torch.float16, device="cuda")

        def call(i):
            Q.qmoe_ragged_mm(X, offs, ws[i % 4], N, E, block, out=Y)

        ku = T.kernel_us([lambda i=i: call(i) for i in range(12)])
        us = ku["kernel_us"]
        used = int((counts > 0).sum())
        res.append({"T": T_, "rows": R, "experts_used": used, "kernel_us": round(us, 2),
                    "TFLOPs": round(2.0 * R * N * K / us / 1e6, 1),
                    "weight_GBps": round(used * per_expert / us / 1e3, 1)})
        del X, Y
    torch.cuda.empty_cache()
    log(f"[ragged] {len(res)} cases")
    return res


def wide_leg(T):
    """MatMulNBits at M = 1 (fp32 A/C, block 64, default zero point) with 3-, 4- and
    8-bit weights at the phi4 gate_up and lm_head shapes, copies >= 1 GiB per shape."""
    import torch
    from gemm_qmm_nbits_amd import qmm as Q
    out = {}
    for bits in (3, 4, 8):
        for name, (K, N) in (("gate_up", (5120, 35840)), ("lm_head", (5120, 100352))):
            b = weight_bytes_nbits(K, N, bits=bits)
            pool = nbits_copies(K, N, bits, pool_copies(b), 6000 + bits)
            A = torch.randn((1, K), device="cuda")
            C = torch.empty((1, N), device="cuda")

            def call(i, A=A, C=C, pool=pool, K=K, bits=bits):
                W, S = pool[i % len(pool)]
                Q.qmm_nbits(A, W, S, K, bits, 64, None, Q.QMM_ZP_NONE, 0.0, out=C)

            n = max(len(pool), 20)
            ku = T.kernel_us([lambda i=i: call(i) for i in range(n)])
            out[f"u{bits} {name}" if bits != 8 else f"i8 {name}"] = {
                "K": K, "N": N, "weight_MB": round(b / 1e6, 2), "kernel_us": round(ku["kernel_us"], 2),
                "GBps": round(b / ku["kernel_us"] / 1e3, 1),
                "frac_hbm": round(b / ku["kernel_us"] / 1e3 / HBM_PEAK_GBS, 4)}
            del pool
            torch.cuda.empty_cache()
    log(f"[wide] {len(out)} cases")
    return out


def qdq_leg(T):
    """Device Q/DQ ops on an fp16 activation tensor of 8192 x 5760 (47.2 M elements):
    fake_quantize (u8) and the fused quantized SwiGLU (gate, up -> out); bytes read +
    written per call over the kernel time."""
    import torch
    from gemm_qmm_nbits_amd import qmm as Q
    n = 8192 * 5760
    x = torch.randn(n, device="cuda").half()
    u = torch.randn(n, device="cuda").half()
    y = torch.empty_like(x)
    q = (0.02, 128)
    qp = [(0.03, 120), (1.0 / 255, 0), (0.02, 20), (0.03, 130), (0.05, 100)]
    res = {}
    ku = T.kernel_us([lambda: Q.fake_quantize(x, q, 8, out=y)] * 10)
    res["fake_quantize fp16 u8"] = {"elements": n, "kernel_us": round(ku["kernel_us"], 2),
                                    "GBps": round(4 * n / ku["kernel_us"] / 1e3, 1)}
    ku = T.kernel_us([lambda: Q.qswiglu(x, u, qp, 8, out=y)] * 10)
    res["qswiglu fp16 u8"] = {"elements": n, "kernel_us": round(ku["kernel_us"], 2),
                              "GBps": round(6 * n / ku["kernel_us"] / 1e3, 1)}
    for r in res.values():
        r["frac_hbm"] = round(r["GBps"] / HBM_PEAK_GBS, 4)
    del x, u, y
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the decode workload
# ---------------------------------------------------------------------------

def _oracle_samples():
    """(name, weight bytes, callable) for the bounded oracle samples: one full decode step
    of the four phi4 layers at M = 1, the tiny u4 GEMV, qkv at M = 2048, the codebook up
    layer at M = 1 and M = 64, one GPT-OSS MoE token and a 128-expert top-8 burst of 8."""
    from gemm_qmm_nbits_amd import inputs as gen
    from oracle import qmm_oracle as O

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def decode_step():
        tot = 0.0
        for si, (name, (K, N)) in enumerate(gen.PHI4_SHAPES.items()):
            p = gen.nbits_problem(1, K, N, 2, 64, seed=gen.config_seed(1, si), zp="none",
                                  scale_range=(0.01, 0.05))
            tot += timed(lambda: O.qmm_nbits(p["A"], "f32", p["W"], 2, K, 64, p["scales"], None, O.ZP_UNIFORM,
                                             uniform_zp=1.5))
            del p
        return tot

    def tiny():
        p = gen.nbits_problem(1, 256, 128, 4, 64, seed=gen.config_seed(0), zp="packed8")
        return timed(lambda: O.qmm_nbits(p["A"], "f32", p["W"], 4, 256, 64, p["scales"], p["zp"], O.ZP_PACKED))

    def qkv_prefill():
        K, N = gen.PHI4_SHAPES["qkv"]
        p = gen.nbits_problem(2048, K, N, 2, 64, seed=gen.config_seed(1, 20), zp="none", scale_range=(0.01, 0.05))
        return timed(lambda: O.qmm_nbits(p["A"], "f32", p["W"], 2, K, 64, p["scales"], None, O.ZP_UNIFORM,
                                         uniform_zp=1.5))

    def codebook_up(M):
        K, N = gen.CODEBOOK_SHAPES["up"]
        p = gen.codebook_problem(M, K, N, seed=gen.config_seed(2, 2))
        return timed(lambda: O.qmm_codebook4(p["A"], "bf16", p["W"], K, 64, p["absmax"], p["codebook"]))

    def moe(T_, c, zp):
        p = gen.qmoe_problem(T_, c["H"], c["I"], c["E"], c["k"], 64, seed=gen.config_seed(3, 1), zp=zp)
        return timed(lambda: O.qmoe_decode(p["X"], p["ids"], p["rw"], p["fc1"], p["fc2"], c["H"], c["I"], 64))

    g, q = gen.QMOE_GPT_OSS, gen.QMOE_128
    moe_b = g["k"] * (weight_bytes_nbits(g["H"], 2 * g["I"], bits=4) + weight_bytes_nbits(g["I"], g["H"], bits=4))
    q_b = 64 * qmoe_bytes(q["H"], q["I"], 64, True, False, 1)
    Kc, Nc = gen.CODEBOOK_SHAPES["up"]
    cb_b = Nc * (Kc // 2) + Nc * (Kc // 64) * 4
    K1, N1 = gen.PHI4_SHAPES["qkv"]
    return [("decode step (qkv, gate_up, down, lm_head; u2, M=1)",
             sum(weight_bytes_nbits(K, N) for K, N in gen.PHI4_SHAPES.values()), decode_step),
            ("tiny u4 GEMV M=1 K=256 N=128", 128 * 4 * (32 + 2) + 128 * 2, tiny),
            ("qkv 5120x7680 u2, M=2048", weight_bytes_nbits(K1, N1), qkv_prefill),
            ("codebook up 4096x14336, M=1", cb_b, lambda: codebook_up(1)),
            ("codebook up 4096x14336, M=64", cb_b, lambda: codebook_up(64)),
            ("GPT-OSS-20B MoE, one token, block 64 (4 experts)", moe_b, lambda: moe(1, g, False)),
            ("128x768 top-8 MoE, T=8, block 64, zp (64 (token, slot) pairs)", q_b, lambda: moe(8, q, True))]


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    """The oracle, as it stands, on bounded samples of the workloads, with one thread and
    with 16 threads (numpy's BLAS threads; 16 is one GPU's share of the host's cores)."""
    from threadpoolctl import threadpool_limits

    host_cores = os.cpu_count()
    allowed = len(os.sched_getaffinity(0))
    many = min(16, allowed)
    runs = {}
    for threads in (1, many):
        res = []
        with threadpool_limits(limits=threads):
            for name, nbytes, fn in _oracle_samples():
                secs = fn()
                res.append({"sample": name, "weight_MB": round(nbytes / 1e6, 3),
                            "s_per_call": round(secs, 4), "GBps": round(nbytes / secs / 1e9, 5)})
        runs[threads] = res
    head = runs[1][0]
    return {"value": head["GBps"], "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one full decode step (qkv, gate_up, down, lm_head at M=1): "
                      f"{head['weight_MB']:.1f} MB of weights in {head['s_per_call']:.1f} s, "
                      f"numpy fp64, 1 thread",
            "cpu_model": _cpu_model(), "host_cores": host_cores, "cores_allowed": allowed,
            "all_cores": {"cores": many, "value": runs[many][0]["GBps"], "unit": "GB/s"},
            "samples": {"1_thread": runs[1], f"{many}_threads": runs[many]}}


def ceilings_leg(T):
    """Achievable ceilings next to the spec peaks: a hand-written streaming read (128-bit
    loads, every byte once) over 4 GiB, at several grid sizes; a device copy (torch) over
    the lm_head weight bytes rotated over 8 buffers; an fp16 matrix product through
    torch.matmul (hipBLASLt) at the phi4 qkv and lm_head shapes, M = 2048."""
    import torch
    from gemm_qmm_nbits_amd import qmm as Q
    out = {}
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    sweep = {}
    for groups in (1024, 2048, 4096, 8192, 16384):
        ku = T.kernel_us([lambda: Q.hbm_read_probe(big, sink, groups)] * 6)
        sweep[groups] = round((4 << 30) / ku["kernel_us"] / 1e3, 1)
    best = max(sweep, key=sweep.get)
    out["stream_read_128b"] = {"bytes": 4 << 30, "GBps_by_workgroups": sweep, "best_GBps": sweep[best],
                               "best_frac_hbm": round(sweep[best] / HBM_PEAK_GBS, 4)}
    # the same read at the sizes of the decode layers and MoE calls: the fixed cost of a
    # launch that streams a few MB, buffers rotated through the 4 GiB so every read is cold
    by_size = {}
    for mb in (2, 4, 11, 20, 26, 53, 145, 512):
        nb = mb * 1000000 // 4096 * 4096
        nbuf = (4 << 30) // nb
        best = None
        for groups in (256, 512, 1024, 2048, 4096):
            views = [big[i * nb:(i + 1) * nb] for i in range(min(nbuf, 64))]
            ku = T.kernel_us([lambda i=i: Q.hbm_read_probe(views[i % len(views)], sink, groups)
                              for i in range(max(16, min(len(views), 64)))])
            if best is None or ku["kernel_us"] < best[1]:
                best = (groups, ku["kernel_us"])
        by_size[mb] = {"workgroups": best[0], "kernel_us": round(best[1], 2),
                       "GBps": round(nb / best[1] / 1e3, 1)}
    out["stream_read_128b"]["by_size_MB"] = by_size
    del big
    torch.cuda.empty_cache()
    nbytes = int(weight_bytes_nbits(5120, 100352)) // 256 * 256
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(8)]
    dsts = [torch.empty_like(b) for b in bufs]
    ku = T.event_us([lambda i=i: dsts[i % 8].copy_(bufs[i % 8]) for i in range(16)])
    out["copy_read_plus_write_GBps"] = round(2 * nbytes / ku["event_us"] / 1e3, 1)
    del bufs, dsts
    torch.cuda.empty_cache()
    mm = {}
    for name, (K, N) in (("qkv", (5120, 7680)), ("lm_head", (5120, 100352))):
        a = torch.randn((2048, K), device="cuda", dtype=torch.float16)
        b = torch.randn((K, N), device="cuda", dtype=torch.float16)
        c = torch.empty((2048, N), device="cuda", dtype=torch.float16)
        us = T.event_us([lambda: torch.matmul(a, b, out=c)] * 5)["event_us"]
        mm[name] = {"M": 2048, "K": K, "N": N, "us": round(us, 1),
                    "TFLOPs": round(2 * 2048 * K * N / us / 1e6, 1)}
        del a, b, c
    out["fp16_matmul_hipblaslt"] = mm
    torch.cuda.empty_cache()
    return out


def n_sweep_leg(T):
    """The 2-bit GEMV (M = 1, K = 5120) at N around the gate_up and lm_head widths, in
    steps of 16 rows, to expose memory-channel outliers; >= 1 GiB of copies per point,
    carved from one pool of random bytes and fp16 scales."""
    import torch
    from gemm_qmm_nbits_amd import qmm as Q
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    K, nblk = 5120, 80
    pool_rows = 800000        # 1.02 GB of codes + 128 MB of scales: >= 7 copies at N = 100k
    Wp = torch.randint(0, 256, (pool_rows, nblk * 16), dtype=torch.uint8, device="cuda", generator=g)
    Sp = (torch.rand((pool_rows, nblk), device="cuda", generator=g) * 0.04 + 0.01).half()
    A = torch.randn((1, K), device="cuda", generator=g)
    res = []
    for N0 in (35840, 100352):
        for d in (-128, -64, -32, -16, 0, 16, 32, 64, 128):
            N = N0 + d
            copies = pool_rows // N
            C = torch.empty((1, N), device="cuda")
            sets = [(Wp[c * N:(c + 1) * N], Sp[c * N:(c + 1) * N]) for c in range(copies)]

            def call(i, sets=sets, C=C):
                W, S = sets[i % len(sets)]
                Q.qmm_nbits(A, W, S, K, 2, 64, None, Q.QMM_ZP_UNIFORM, 1.5, out=C)

            ku = T.kernel_us([lambda i=i: call(i) for i in range(max(copies, 12))])
            b = weight_bytes_nbits(K, N)
            res.append({"N": N, "kernel_us": round(ku["kernel_us"], 2),
                        "GBps": round(b / ku["kernel_us"] / 1e3, 1)})
    del Wp, Sp
    torch.cuda.empty_cache()
    return res


def copy_calibration(nbytes=256 << 20, calls=5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(calls):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_per_copy": nbytes, "calls": calls}


def roofline_entry(dec):
    """Dominant kernel of the decode step: the lm_head GEMV (62% of the step's bytes).
    `achieved` = its algorithmic bytes per launch / its mean launch time from one event
    pair per launch; the committed kernel-trace mean of the same kernel is carried next to
    it when the trace was taken on the current kernel sources."""
    if "lm_head" not in dec["shapes"]:
        return None
    lm = dec["shapes"]["lm_head"]
    b = int(weight_bytes_nbits(5120, 100352))
    achieved = b / lm["kernel_us"] / 1e3
    r = {"bound": "hbm", "kernel": "gemv_ip_stream_kernel (u2, fp32 A, M=1) on lm_head 5120x100352",
         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("gemv_lm_head"),
         "algorithmic_bytes_per_launch": b, "avg_launch_us": lm["kernel_us"],
         "graph_back_to_back_us": lm["graph_us"]}
    tr = trace_mean("gemv_lm_head")
    if tr is not None:
        r["trace_avg_launch_us"] = tr
        r["trace_frac"] = round(b / tr / 1e3 / HBM_PEAK_GBS, 4)
    return r


def _profile_entry(fname, key):
    """Entry `key` of a committed profile summary (JSON) if its kernel sources are unchanged."""
    import hashlib
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    h = hashlib.sha256()
    for rel in t.get("sources", []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != t.get("sources_sha256"):
        return None
    return t.get("kernels", {}).get(key)


def trace_mean(key):
    e = _profile_entry("kernel_means.json", key)
    return None if e is None else e.get("avg_us")


def measured_traffic(key):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources (FETCH_SIZE and WRITE_SIZE, each x its copy-kernel factor)."""
    e = _profile_entry("traffic.json", key)
    return None if e is None else e.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(the per-GPU shard of a multi-GPU run is the same kernel at N/G)"}))
        sys.exit(2)
    import torch
    from gemm_qmm_nbits_amd import qmm as Q

    torch.cuda.set_device(0)
    Q.lib()
    legs = set(args.legs.split(","))
    T = Timer()
    dec = decode_leg(args, T)
    value = dec["step_bytes"] / (dec["step_ms"] * 1e-3) / 1e9
    out = {
        "metric": "weight GB/s & % HBM peak at M=1..64; prefill TFLOP/s; QMoE decode tok/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u2 weights x fp32 activations: A as 23-bit block fixed point per scale group, "
                 "int32 dot, fp32 accumulate",
        "data": "synthetic (seeded random codes, scales and activations of the phi4-14B 2-bit shapes)",
        "config": {"workload": "phi4-14B-shaped 2-bit MatMulNBits decode, M=1, block 64, uniform zp 1.5, "
                               "fp32 A/C: qkv 5120x7680, gate_up 5120x35840, down 17920x5120, "
                               "lm_head 5120x100352",
                   "M": 1, "bits": 2, "block": 64,
                   "weight_copies_per_shape": {k: v["copies"] for k, v in dec["shapes"].items()}},
        "roofline": roofline_entry(dec),
        "decode_shapes": dec["shapes"],
        "decode_steps_per_graph": dec["steps_per_graph"],
        "ms_per_step_one_step_graphs": round(dec["step_ms_one_step_graphs"], 4),
        "graph_replay_matches_eager": dec["graph_replay_matches_eager"],
    }
    if "tiny" in legs:
        out["tiny_u4"] = tiny_leg(T)
    if "prefill" in legs:
        out["prefill"] = prefill_leg(args)
    if "stack" in legs:
        out["phi4_stack"] = stack_leg(args)
    if "codebook" in legs:
        out["codebook"] = codebook_leg(T)
    if "wide" in legs:
        out["wide_codes"] = wide_leg(T)
    if "ragged" in legs:
        out["ragged_mm"] = ragged_leg(T)
    if "qdq" in legs:
        out["qdq"] = qdq_leg(T)
    if "copycal" in legs:
        out["copy_calibration"] = copy_calibration()
    if "ceilings" in legs:
        out["ceilings"] = ceilings_leg(T)
    if "nsweep" in legs:
        out["n_sweep"] = n_sweep_leg(T)
    if "qmoe" in legs:
        out["qmoe"] = qmoe_legs(T)
    T.release()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
