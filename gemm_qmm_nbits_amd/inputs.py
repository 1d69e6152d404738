"""Seeded synthetic inputs for the low-bit dequantize-matmul path.

This module only draws random data.  It holds none of the method's arithmetic:
packed weights are drawn directly as uniform random bytes (so every 2- or 4-bit
code inside them is i.i.d. uniform), zero points as bytes or fp16 fills, and
floating values are drawn in fp64 and rounded to the stated storage dtype by
numpy/torch casts.  Both the oracle-side tests and the GPU-side tests and bench
take their inputs from here; nothing here imports the oracle or the HIP library.

Storage conventions (the problem statement of the MatMulNBits pages: A[M,K],
packed W[N,K] along K with block size B, per-block fp16 scales, zero point
tensor or uniform scalar):
  * W        uint8 [N, nblk, B*bits/8]  nblk = ceil(K/B); ragged tail bytes are
             random (a correct consumer never reads past K)
  * scales   uint16 fp16 bits [N, nblk]
  * zp       packed: uint8 [N, ceil(nblk*bits/8)]; fp16: uint16 [N, nblk]
  * bf16 / fp16 activations are stored as uint16 bit patterns; fp32 as float32.
"""
from __future__ import annotations

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def config_seed(config_index: int, shape_index: int = 0) -> int:
    """Seed recipe: 1000*(config+1) + shape index."""
    return 1000 * (config_index + 1) + shape_index


def nblocks(K: int, block: int) -> int:
    return (K + block - 1) // block


def _f16_bits(x64: np.ndarray) -> np.ndarray:
    return np.asarray(x64, dtype=np.float64).astype(np.float16).view(np.uint16)


def _bf16_bits(x64: np.ndarray) -> np.ndarray:
    import torch  # library cast fp32 -> bf16 (round to nearest even)

    t = torch.from_numpy(np.asarray(x64, dtype=np.float64).astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def activations(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) activations drawn in fp64, rounded to `dtype` storage."""
    x = rng.standard_normal(shape)
    if dtype == F32:
        return x.astype(np.float32)
    if dtype == F16:
        return _f16_bits(x)
    if dtype == BF16:
        return _bf16_bits(x)
    raise ValueError(dtype)


def packed_weights(rng, N: int, K: int, bits: int, block: int, lead=()) -> np.ndarray:
    blob = block * bits // 8
    return rng.integers(0, 256, size=tuple(lead) + (N, nblocks(K, block), blob),
                        dtype=np.uint8)


def fp16_uniform(rng, shape, lo: float, hi: float) -> np.ndarray:
    return _f16_bits(rng.uniform(lo, hi, size=shape))


def packed_zero_points(rng, N: int, nblk: int, bits: int, fill: int | None = None,
                       lead=()) -> np.ndarray:
    """Packed unsigned zero points, one `bits`-wide code per (row, block).

    fill=None draws uniform random bytes (i.e. i.i.d. uniform codes); an integer
    fill replicates that code in every field of every byte (e.g. 8 -> 0x88 for
    4-bit codes).
    """
    nbytes = (nblk * bits + 7) // 8
    shape = tuple(lead) + (N, nbytes)
    if fill is None:
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    # the code `fill` in every field of a row's little-endian bit stream
    bits_row = np.zeros(nbytes * 8 + 8, dtype=np.uint8)
    for b in range(nblk):
        for i in range(bits):
            bits_row[b * bits + i] = (fill >> i) & 1
    row = np.packbits(bits_row[: nbytes * 8].reshape(nbytes, 8), axis=1, bitorder="little").ravel()
    return np.broadcast_to(row, shape).copy()


def fp16_fill(shape, value: float) -> np.ndarray:
    return _f16_bits(np.full(shape, value))


def codebook16(rng) -> np.ndarray:
    """16-entry sorted fp32 codebook in [-1, 1] containing -1, 0 and 1.

    The other 13 entries are i.i.d. U(-1, 1) draws, rejecting exact zeros and
    duplicates, rounded to fp32.
    """
    vals = {np.float32(-1.0), np.float32(0.0), np.float32(1.0)}
    while len(vals) < 16:
        v = np.float32(rng.uniform(-1.0, 1.0))
        if v != 0.0:
            vals.add(v)
    return np.array(sorted(vals), dtype=np.float32)


def fp32_uniform(rng, shape, lo: float, hi: float) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def nested_absmax_inputs(rng, N: int, nblk: int, group: int = 256):
    """Double-quantized absmax storage: uint8 codes [N][nblk] (uniform), a sorted
    256-entry fp32 table in [-1, 1] holding -1, 0 and 1 (the other entries i.i.d.
    U(-1, 1), no repeats), fp32 scales U[0.01, 0.04] per `group` blocks and an fp32
    offset 0.055 (so the decoded absmax lies in [0.015, 0.095])."""
    codes = rng.integers(0, 256, size=(N, nblk), dtype=np.uint8)
    vals = {np.float32(-1.0), np.float32(0.0), np.float32(1.0)}
    while len(vals) < 256:
        v = np.float32(rng.uniform(-1.0, 1.0))
        if v != 0.0:
            vals.add(v)
    table = np.array(sorted(vals), dtype=np.float32)
    ngroups = (N * nblk + group - 1) // group
    scales = rng.uniform(0.01, 0.04, size=ngroups).astype(np.float32)
    return {"codes": codes, "table": table, "scales": scales, "offset": np.float32(0.055), "group": group}


def routing(rng, T: int, E: int, k: int):
    """Top-k routing from N(0,1) logits: ids [T,k] int32, weights [T,k] fp32.

    The k largest logits are taken (ties to the lower expert index, in
    descending logit order) and their weights are a softmax over those k.
    """
    logits = rng.standard_normal((T, E))
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        sel = logits[t, order]
        ex = np.exp(sel - sel.max())
        ids[t] = order
        w[t] = (ex / ex.sum()).astype(np.float32)
    return ids, w


# ---------------------------------------------------------------------------
# Problem bundles with the shapes and distributions of the five workloads.
# ---------------------------------------------------------------------------

def nbits_problem(M, K, N, bits, block, *, seed, a_dtype=F32, scale_range=(0.005, 0.02),
                  zp="packed8", uniform_zp=1.5, bias=False):
    """One MatMulNBits problem.

    zp: "packed8" (packed code 2^(bits-1) everywhere), "packed" (random codes),
        "f16_uniform" (fp16 tensor filled with `uniform_zp`), "f16" (random fp16
        in [0, 2^bits - 1], or [-8, 8] for signed 8-bit codes) or "none".
    Draw order: A, codes, scales, zero points, bias.
    """
    rng = make_rng(seed)
    nblk = nblocks(K, block)
    p = {"M": M, "K": K, "N": N, "bits": bits, "block": block, "a_dtype": a_dtype,
         "seed": seed, "zp_mode": zp}
    p["A"] = activations(rng, (M, K), a_dtype)
    p["W"] = packed_weights(rng, N, K, bits, block)
    p["scales"] = fp16_uniform(rng, (N, nblk), *scale_range)
    if zp == "packed8":
        p["zp"] = packed_zero_points(rng, N, nblk, bits, fill=1 << (bits - 1))
    elif zp == "packed":
        p["zp"] = packed_zero_points(rng, N, nblk, bits)
    elif zp == "f16_uniform":
        p["zp"] = fp16_fill((N, nblk), uniform_zp)
        p["uniform_zp"] = float(np.float16(uniform_zp))
    elif zp == "f16":
        lo, hi = (-8.0, 8.0) if bits == 8 else (0.0, float((1 << bits) - 1))
        p["zp"] = fp16_uniform(rng, (N, nblk), lo, hi)
    elif zp == "none":
        p["zp"] = None
    else:
        raise ValueError(zp)
    p["bias"] = activations(rng, (N,), F32) if bias else None
    return p


def codebook_problem(M, K, N, *, seed, a_dtype=BF16, block=64, absmax_range=(0.01, 0.1),
                     bias=False):
    """One 16-entry-codebook 4-bit problem.  Draw order: A, codes, codebook, absmax."""
    rng = make_rng(seed)
    nblk = nblocks(K, block)
    p = {"M": M, "K": K, "N": N, "block": block, "a_dtype": a_dtype, "seed": seed}
    p["A"] = activations(rng, (M, K), a_dtype)
    p["W"] = packed_weights(rng, N, K, 4, block)
    p["codebook"] = codebook16(rng)
    p["absmax"] = fp32_uniform(rng, (N, nblk), *absmax_range)
    p["bias"] = activations(rng, (N,), a_dtype) if bias else None
    return p


def qmoe_problem(T, H, I, E, k, block, *, seed, zp=False, bias=False,
                 scale_range=(0.005, 0.02), bits=4):
    """One fused-MoE decode problem (fc1 [E][2I][H], fc2 [E][H][I], u4).

    Draw order: X, routing logits, fc1 codes, fc1 scales, fc1 zp, fc1 bias,
    fc2 codes, fc2 scales, fc2 zp, fc2 bias.
    """
    rng = make_rng(seed)
    p = {"T": T, "H": H, "I": I, "E": E, "k": k, "block": block, "bits": bits, "seed": seed}
    p["X"] = activations(rng, (T, H), F16)
    p["ids"], p["rw"] = routing(rng, T, E, k)
    for name, n_out, k_in in (("fc1", 2 * I, H), ("fc2", H, I)):
        nblk = nblocks(k_in, block)
        d = {"W": packed_weights(rng, n_out, k_in, bits, block, lead=(E,)),
             "scales": fp16_uniform(rng, (E, n_out, nblk), *scale_range)}
        d["zp"] = packed_zero_points(rng, n_out, nblk, bits, lead=(E,)) if zp else None
        d["bias"] = activations(rng, (E, n_out), F16) if bias else None
        p[name] = d
    return p


# Shapes of the five workloads.
PHI4_SHAPES = {"qkv": (5120, 7680), "gate_up": (5120, 35840), "down": (17920, 5120),
               "lm_head": (5120, 100352)}
CODEBOOK_SHAPES = {"gqa_kv": (4096, 1024), "square": (4096, 4096), "up": (4096, 14336),
                   "moe_down": (1536, 4096)}
CODEBOOK_M = (1, 4, 16, 64)
QMOE_GPT_OSS = {"E": 32, "k": 4, "H": 2880, "I": 2880}
QMOE_128 = {"E": 128, "k": 8, "H": 2048, "I": 768, "block": 64}
