"""Benchmark of the fused low-bit dequantize-matmul path on one MI355X.

One step = one decode pass (M = 1) over the four phi4-14B-shaped 2-bit
MatMulNBits layers (qkv 5120x7680, gate_up 5120x35840, down 17920x5120,
lm_head 5120x100352; block 64, fp16 scales, uniform zero point 1.5, fp32 A and
C).  Weights are resident in HBM and rotated through enough copies (>= 1 GiB,
four times the 256 MB last-level cache) that every step reads them cold.
`value` is the weight bytes streamed per step divided by the step time.

Extra legs in the same JSON line: the fused MoE decode (GPT-OSS-20B shape and
the 128-expert top-8 shape, fresh routing per call) and the prefill matmul when
built.  Each kernel launch is bracketed by HIP events on the stream it runs on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
    ap.add_argument("--legs", default="decode,stack,prefill,qmoe,codebook,ceilings",
                    help="comma list of decode,stack,prefill,qmoe,codebook,ceilings "
                         "(copycal: a plain copy for counter calibration; nsweep: the GEMV "
                         "at N around the gate_up and lm_head widths)")
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
# decode leg: phi4 2-bit M = 1
# ---------------------------------------------------------------------------

def decode_leg(args):
    """Decode step = the four phi4 layers at M = 1, captured as one HIP graph per
    weight copy and replayed back to back (launch gaps of the host excluded)."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q

    want = args.decode_shapes.split(",")
    shapes = [(n, kn) for n, kn in gen.PHI4_SHAPES.items() if n in want]
    step_bytes = sum(weight_bytes_nbits(K, N) for _, (K, N) in shapes)
    copies = max(2, int(np.ceil(1.0 * (1 << 30) / step_bytes)) + 1)
    log(f"[decode] {len(shapes)} shapes, {step_bytes / 1e6:.1f} MB weights/step, {copies} copies")
    sets = []
    for ci in range(copies):
        layer = []
        for name, (K, N) in shapes:
            si = list(gen.PHI4_SHAPES).index(name)
            p = gen.nbits_problem(1, K, N, 2, 64, seed=gen.config_seed(1, si) + 100 * ci,
                                  zp="none", scale_range=(0.01, 0.05))
            layer.append({"name": name, "K": K, "N": N, "A": to_dev(p["A"]), "W": to_dev(p["W"]),
                          "scales": to_dev(p["scales"]),
                          "C": torch.empty((1, N), dtype=torch.float32, device="cuda")})
        sets.append(layer)

    def launch(L):
        Q.qmm_nbits(L["A"], L["W"], L["scales"], L["K"], 2, 64, None, Q.QMM_ZP_UNIFORM, 1.5,
                    out=L["C"])

    # eager warm-up: the first call of each shape runs the up-front tiling choice
    for layer in sets:
        for L in layer:
            launch(L)
    torch.cuda.synchronize()
    eager_ref = [L["C"].clone() for L in sets[0]]
    cap = torch.cuda.Stream()
    step_graphs = []
    with torch.cuda.stream(cap):
        for layer in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for L in layer:
                    launch(L)
            step_graphs.append(g)
        # one graph per shape: that layer of every copy, back to back (cold rotation)
        shape_graphs = []
        for j in range(len(shapes)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for layer in sets:
                    launch(layer[j])
            shape_graphs.append(g)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step_graphs[i % copies].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step_graphs[i % copies].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    shapes_out = {}
    reps = 5
    for j, (name, (K, N)) in enumerate(shapes):
        shape_graphs[j].replay()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(reps):
            shape_graphs[j].replay()
        a1.record(stream)
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) * 1e3 / (reps * copies)
        b = weight_bytes_nbits(K, N)
        shapes_out[name] = {"K": K, "N": N, "weight_MB": round(b / 1e6, 3), "us": round(us, 2),
                            "GBps": round(b / (us * 1e-6) / 1e9, 1),
                            "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    # the decode outputs of the graph replays equal the eager ones
    for L in sets[0]:
        L["C"].zero_()
    step_graphs[0].replay()
    torch.cuda.synchronize()
    same = all(torch.equal(r, L["C"]) for r, L in zip(eager_ref, sets[0]))
    return {"step_bytes": step_bytes, "step_ms": step_ms, "wall_s": wall, "shapes": shapes_out,
            "copies": copies, "graph_replay_matches_eager": bool(same)}


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

def codebook_leg(args, reps=5):
    """Weight GB/s of qmm_codebook4 at the four codebook shapes for M = 1, 4, 16, 64:
    bf16 A and C, block 64, weights rotated over copies >= 1 GiB, each shape's calls
    captured in one HIP graph (M = 1: weight-streaming GEMV; M >= 4: matrix cores)."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q

    out = {}
    stream = torch.cuda.current_stream()
    for name, (K, N) in gen.CODEBOOK_SHAPES.items():
        nblk = (K + 63) // 64
        wbytes = N * nblk * (32 + 4)  # packed codes + fp32 absmax
        copies = max(2, int(np.ceil((1 << 30) / wbytes)) + 1)
        base = gen.codebook_problem(1, K, N, seed=gen.config_seed(2, 1000 + list(gen.CODEBOOK_SHAPES).index(name)))
        cb = to_dev(base["codebook"])
        g = torch.Generator(device="cuda")
        g.manual_seed(N)
        Ws = [torch.randint(0, 256, (N, nblk * 32), dtype=torch.uint8, device="cuda", generator=g)
              for _ in range(copies)]
        ams = [(torch.rand((N, nblk), device="cuda", generator=g) * 0.09 + 0.01) for _ in range(copies)]
        for M in gen.CODEBOOK_M:
            A = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
            C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            wsb = Q.lib().qmm_codebook4_workspace_bytes(M, K, N, Q.QMM_BF16)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

            def call(i):
                Q.qmm_codebook4(A, Ws[i], ams[i], cb, K, 64, None, out=C, workspace=ws if wsb else None)

            for i in range(copies):
                call(i)
            torch.cuda.synchronize()
            cap = torch.cuda.Stream()
            with torch.cuda.stream(cap):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=cap):
                    for i in range(copies):
                        call(i)
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
            gbs = wbytes / (us * 1e-6) / 1e9
            out[f"{name} M={M}"] = {"K": K, "N": N, "M": M, "us": round(us, 2), "weight_GBps": round(gbs, 1),
                                    "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                    "path": "gemv" if M < 4 else "matrix cores"}
            del gr
        del Ws, ams
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


def qmoe_leg(args, name, T, H, I, E, k, block, zp, bias, mode, calls=48):
    """Fused MoE decode: `calls` calls with fresh routing each and whole-layer weight
    copies rotated (>= 1 GiB), captured in one HIP graph and replayed; mean per call."""
    import torch
    from gemm_qmm_nbits_amd import inputs as gen
    from gemm_qmm_nbits_amd import qmm as Q

    layer_bytes = qmoe_bytes(H, I, block, zp, bias, E)
    copies = max(2, int(np.ceil((1 << 30) / layer_bytes)))
    p = gen.qmoe_problem(T, H, I, E, k, block, seed=gen.config_seed(3 if E == 32 else 4, T),
                         zp=zp, bias=bias)
    fcs = []
    for c in range(copies):
        d = {}
        for fc in ("fc1", "fc2"):
            src = p[fc]
            d[fc] = {"W": to_dev(src["W"]), "scales": to_dev(src["scales"]),
                     "zp": to_dev(src["zp"]) if src["zp"] is not None else None,
                     "bias": to_dev(src["bias"]) if src["bias"] is not None else None}
        fcs.append(d)
    X = to_dev(p["X"]).view(torch.float16)
    rng = np.random.default_rng(7)
    routes = []
    n_unique = []
    for i in range(calls):
        ids, w = gen.routing(rng, T, E, k)
        routes.append((to_dev(ids), to_dev(w)))
        n_unique.append(len(np.unique(ids)))
    Y = torch.empty((T, H), dtype=torch.float16, device="cuda")
    scratch = torch.zeros(Q.qmoe_decode_scratch_bytes(T, H, I, k, mode), dtype=torch.uint8,
                          device="cuda")

    def call(i):
        d = fcs[i % copies]
        Q.qmoe_decode_fused(X, routes[i][0], routes[i][1], d["fc1"], d["fc2"], H, I, E, block,
                            mode=mode, out=Y, scratch=scratch)

    for i in range(min(calls, 4)):   # eager: the first call times the tiling candidates
        call(i)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(calls):
                call(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * calls)
    uniq = float(np.mean(n_unique))
    per_expert = qmoe_bytes(H, I, block, zp, bias, 1)
    gbps = uniq * per_expert / (us * 1e-6) / 1e9
    del fcs, g
    torch.cuda.empty_cache()
    return {"name": name, "T": T, "H": H, "I": I, "E": E, "k": k, "block": block, "zp": zp,
            "bias": bias, "mode": "int8" if mode == Q.QMOE_INT8_ACT else "fp",
            "us_per_call": round(us, 2), "tok_per_s": round(T / (us * 1e-6), 1),
            "weight_MB_per_call": round(uniq * per_expert / 1e6, 2),
            "weight_GBps": round(gbps, 1), "frac_hbm": round(gbps / HBM_PEAK_GBS, 4),
            "unique_experts_mean": uniq}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the decode workload
# ---------------------------------------------------------------------------

def _oracle_samples():
    """(name, weight bytes, callable) for the bounded oracle samples: one full decode step
    of the four phi4 layers at M = 1, one codebook layer at M = 1, one MoE token."""
    from gemm_qmm_nbits_amd import inputs as gen
    from oracle import qmm_oracle as O

    def decode_step():
        for si, (name, (K, N)) in enumerate(gen.PHI4_SHAPES.items()):
            p = gen.nbits_problem(1, K, N, 2, 64, seed=gen.config_seed(1, si), zp="none",
                                  scale_range=(0.01, 0.05))
            t0 = time.perf_counter()
            O.qmm_nbits(p["A"], "f32", p["W"], 2, K, 64, p["scales"], None, O.ZP_UNIFORM,
                        uniform_zp=1.5)
            yield time.perf_counter() - t0
            del p

    def codebook_up():
        K, N = gen.CODEBOOK_SHAPES["up"]
        p = gen.codebook_problem(1, K, N, seed=gen.config_seed(2, 2))
        t0 = time.perf_counter()
        O.qmm_codebook4(p["A"], "bf16", p["W"], K, 64, p["absmax"], p["codebook"])
        yield time.perf_counter() - t0

    def moe_token():
        c = gen.QMOE_GPT_OSS
        p = gen.qmoe_problem(1, c["H"], c["I"], c["E"], c["k"], 64, seed=gen.config_seed(3, 1))
        t0 = time.perf_counter()
        O.qmoe_decode(p["X"], p["ids"], p["rw"], p["fc1"], p["fc2"], c["H"], c["I"], 64)
        yield time.perf_counter() - t0

    c = gen.QMOE_GPT_OSS
    moe_b = c["k"] * (weight_bytes_nbits(c["H"], 2 * c["I"], bits=4) +
                      weight_bytes_nbits(c["I"], c["H"], bits=4))
    Kc, Nc = gen.CODEBOOK_SHAPES["up"]
    return [("decode step (qkv, gate_up, down, lm_head; u2, M=1)",
             sum(weight_bytes_nbits(K, N) for K, N in gen.PHI4_SHAPES.values()), decode_step),
            ("codebook up 4096x14336, M=1", Nc * (Kc // 2) + Nc * (Kc // 64) * 4, codebook_up),
            ("GPT-OSS-20B MoE, one token, block 64 (4 experts)", moe_b, moe_token)]


def cpu_baseline():
    """The oracle, as it stands, on bounded samples of the workloads, with one thread and
    with the host's cores (numpy's BLAS threads; capped at 16, one GPU's share of a host)."""
    from threadpoolctl import threadpool_limits

    all_cores = min(16, len(os.sched_getaffinity(0)))
    runs = {}
    for threads in (1, all_cores):
        res = []
        with threadpool_limits(limits=threads):
            for name, nbytes, fn in _oracle_samples():
                secs = sum(fn())
                res.append({"sample": name, "weight_MB": round(nbytes / 1e6, 3),
                            "s_per_call": round(secs, 4), "GBps": round(nbytes / secs / 1e9, 4)})
        runs[threads] = res
    head = runs[1][0]
    return {"value": head["GBps"], "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one full decode step (qkv, gate_up, down, lm_head at M=1): "
                      f"{head['weight_MB']:.1f} MB of weights in {head['s_per_call']:.1f} s, "
                      f"numpy fp64, 1 thread",
            "all_cores": {"cores": all_cores, "value": runs[all_cores][0]["GBps"], "unit": "GB/s"},
            "samples": {"1_thread": runs[1], f"{all_cores}_threads": runs[all_cores]}}


def ceilings_leg(reps=20):
    """Achievable ceilings on this GPU, next to the spec peaks: a device copy and a
    sum reduction (torch kernels) over the lm_head weight bytes, rotated over copies
    that together exceed the last-level cache, and an fp16 matrix product through
    torch.matmul (hipBLASLt) at the phi4 qkv and lm_head shapes, M = 2048."""
    import torch
    nbytes = int(weight_bytes_nbits(5120, 100352)) // 256 * 256
    copies = 8
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    dsts = [torch.empty_like(b) for b in bufs]
    out = {"bytes": nbytes}
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for i in range(copies):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i % copies)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n  # us per call

    us = timed(lambda i: dsts[i].copy_(bufs[i]), reps)
    out["copy_read_plus_write_GBps"] = round(2 * nbytes / (us * 1e-6) / 1e9, 1)
    views = [b.view(torch.int64) for b in bufs]
    us = timed(lambda i: views[i].sum(), reps)
    out["sum_read_GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    del bufs, dsts, views
    mm = {}
    for name, (K, N) in (("qkv", (5120, 7680)), ("lm_head", (5120, 100352))):
        a = torch.randn((2048, K), device="cuda", dtype=torch.float16)
        b = torch.randn((K, N), device="cuda", dtype=torch.float16)
        c = torch.empty((2048, N), device="cuda", dtype=torch.float16)
        us = timed(lambda i: torch.matmul(a, b, out=c), 5)
        mm[name] = {"M": 2048, "K": K, "N": N, "us": round(us, 1),
                    "TFLOPs": round(2 * 2048 * K * N / (us * 1e-6) / 1e12, 1)}
        del a, b, c
    out["fp16_matmul_hipblaslt"] = mm
    torch.cuda.empty_cache()
    return out


def n_sweep_leg(reps=5, copies=3):
    """The 2-bit GEMV (M = 1, K = 5120) at N around the gate_up and lm_head widths, in
    steps of 16 rows, to expose memory-channel outliers."""
    import torch
    from gemm_qmm_nbits_amd import qmm as Q
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    res = []
    stream = torch.cuda.current_stream()
    for N0 in (35840, 100352):
        for d in (-128, -64, -32, -16, 0, 16, 32, 64, 128):
            N, K = N0 + d, 5120
            sets = []
            for _ in range(copies):
                W = torch.randint(0, 256, (N, 80 * 16), dtype=torch.uint8, device="cuda", generator=g)
                S = (torch.rand((N, 80), device="cuda", generator=g) * 0.04 + 0.01).half()
                A = torch.randn((1, K), device="cuda", generator=g)
                C = torch.empty((1, N), device="cuda")
                sets.append((A, W, S, C))
            for (A, W, S, C) in sets:   # first call of the shape: up-front tiling choice
                Q.qmm_nbits(A, W, S, K, 2, 64, None, Q.QMM_ZP_UNIFORM, 1.5, out=C)
            torch.cuda.synchronize()
            cap = torch.cuda.Stream()
            with torch.cuda.stream(cap):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=cap):
                    for (A, W, S, C) in sets:
                        Q.qmm_nbits(A, W, S, K, 2, 64, None, Q.QMM_ZP_UNIFORM, 1.5, out=C)
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
            b = weight_bytes_nbits(K, N)
            res.append({"N": N, "us": round(us, 2), "GBps": round(b / (us * 1e-6) / 1e9, 1)})
            del sets, gr
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
    """Dominant kernel of the decode step: the lm_head GEMV (62% of the step's bytes)."""
    if "lm_head" not in dec["shapes"]:
        return None
    lm = dec["shapes"]["lm_head"]
    achieved = lm["GBps"]
    r = {"bound": "hbm", "kernel": "gemv_ip_stream_kernel (u2, fp32 A, M=1) on lm_head 5120x100352",
         "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
         "algorithmic_bytes_per_launch": int(weight_bytes_nbits(5120, 100352)),
         "avg_launch_us": lm["us"]}
    r["traffic"] = measured_traffic("gemv_lm_head")
    return r


def measured_traffic(key):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources (FETCH_SIZE x its copy-kernel factor + WRITE_SIZE)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
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
    e = t.get("kernels", {}).get(key)
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
    dec = decode_leg(args)
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
        "dtype": "u2 weights x fp32 activations, fp32 accumulate",
        "data": "synthetic (seeded random codes, scales and activations of the phi4-14B 2-bit shapes)",
        "config": {"workload": "phi4-14B-shaped 2-bit MatMulNBits decode, M=1, block 64, uniform zp 1.5, "
                               "fp32 A/C: qkv 5120x7680, gate_up 5120x35840, down 17920x5120, "
                               "lm_head 5120x100352",
                   "M": 1, "bits": 2, "block": 64, "weight_copies_rotated": dec["copies"]},
        "roofline": roofline_entry(dec),
        "decode_shapes": dec["shapes"],
    }
    if "prefill" in legs:
        out["prefill"] = prefill_leg(args)
    if "stack" in legs:
        out["phi4_stack"] = stack_leg(args)
    if "codebook" in legs:
        out["codebook"] = codebook_leg(args)
    if "copycal" in legs:
        out["copy_calibration"] = copy_calibration()
    if "ceilings" in legs:
        out["ceilings"] = ceilings_leg()
    if "nsweep" in legs:
        out["n_sweep"] = n_sweep_leg()
    if "qmoe" in legs:
        q = []
        q.append(qmoe_leg(args, "gpt-oss-20b", 1, 2880, 2880, 32, 4, 64, False, False, Q.QMOE_FP))
        q.append(qmoe_leg(args, "gpt-oss-20b", 1, 2880, 2880, 32, 4, 64, False, False, Q.QMOE_INT8_ACT))
        for T in (1, 4, 8):
            q.append(qmoe_leg(args, "128x768 top-8", T, 2048, 768, 128, 8, 64, True, False, Q.QMOE_FP))
        out["qmoe"] = q
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
