"""Helpers for the GPU parity tests: move generated problems to the device and
call the C ABI through the binding.  No arithmetic of the method lives here."""
from __future__ import annotations

import sys

import numpy as np

from gemm_qmm_nbits_amd import qmm as Q

# tolerances of the output gates (relative L2 against the fp64 oracle)
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def dev(x):
    """numpy -> cuda tensor (uint16 arrays stay int16 bit patterns)."""
    t = torch()
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return t.from_numpy(x.view(np.int16)).cuda()
    if x.dtype == np.uint32:
        return t.from_numpy(x.view(np.int32)).cuda()
    return t.from_numpy(x).cuda()


def dev_act(x, dtype: str):
    """Activation storage -> cuda tensor of the matching torch dtype."""
    t = torch()
    if dtype == "f32":
        return dev(np.asarray(x, dtype=np.float32))
    td = t.float16 if dtype == "f16" else t.bfloat16
    return dev(np.asarray(x, dtype=np.uint16)).view(td)


def host_f64(t_):
    """cuda tensor (fp32 / fp16 / bf16) -> numpy fp64."""
    tt = torch()
    return t_.detach().to(tt.float64).cpu().numpy()


def host_bits(t_):
    tt = torch()
    if t_.element_size() == 4:
        return t_.detach().view(tt.int32).cpu().numpy()
    return t_.detach().view(tt.int16).cpu().numpy()


ZP_KIND = {"packed8": Q.QMM_ZP_PACKED, "packed": Q.QMM_ZP_PACKED, "f16_uniform": Q.QMM_ZP_F16,
           "f16": Q.QMM_ZP_F16, "none": Q.QMM_ZP_NONE}


def oracle_zp_kind(O, mode):
    return {"packed8": O.ZP_PACKED, "packed": O.ZP_PACKED, "f16_uniform": O.ZP_F16,
            "f16": O.ZP_F16, "none": O.ZP_NONE}[mode]


class NbitsDev:
    """A generated MatMulNBits problem resident on the GPU."""

    def __init__(self, p, c_dtype=None):
        self.p = p
        self.A = dev_act(p["A"], p["a_dtype"])
        self.W = dev(p["W"])
        self.scales = dev(p["scales"])
        self.zp = dev(p["zp"]) if p["zp"] is not None else None
        self.c_dtype = c_dtype or p["a_dtype"]
        tt = torch()
        od = {"f32": tt.float32, "f16": tt.float16, "bf16": tt.bfloat16}[self.c_dtype]
        # the generator draws the bias in fp32; it is stored in the output dtype
        self.bias = (tt.from_numpy(np.asarray(p["bias"], dtype=np.float32)).to(od).cuda()
                     if p["bias"] is not None else None)

    def run(self, uniform=False, out=None, A=None):
        p = self.p
        tt = torch()
        od = {"f32": tt.float32, "f16": tt.float16, "bf16": tt.bfloat16}[self.c_dtype]
        if uniform:
            return Q.qmm_nbits(self.A if A is None else A, self.W, self.scales, p["K"], p["bits"],
                               p["block"], None, Q.QMM_ZP_UNIFORM, p["uniform_zp"], self.bias,
                               out=out, out_dtype=od)
        return Q.qmm_nbits(self.A if A is None else A, self.W, self.scales, p["K"], p["bits"],
                           p["block"], self.zp, ZP_KIND[p["zp_mode"]], 0.0, self.bias, out=out,
                           out_dtype=od)

    def oracle(self, O, rows=None, a_round=None, w_round=None):
        p = self.p
        bias = p["bias"]
        bias_dtype = self.c_dtype
        if bias is not None and self.c_dtype != "f32":
            bias = host_bits(self.bias).view(np.uint16)
        return O.qmm_nbits(p["A"], p["a_dtype"], p["W"], p["bits"], p["K"], p["block"], p["scales"],
                           p["zp"], oracle_zp_kind(O, p["zp_mode"]), 0.0, bias, bias_dtype,
                           a_round=a_round, w_round=w_round, rows=rows)


def sample_rows(N, count, seed):
    """Sorted sample of output columns: the first and last few plus random ones."""
    rng = np.random.default_rng(seed)
    if N <= count:
        return np.arange(N)
    edge = np.r_[0:8, N - 8:N]
    rnd = rng.choice(N, size=count - len(edge), replace=False)
    return np.unique(np.r_[edge, rnd])


# ---------------------------------------------------------------------------
# Per-element bounds next to the relative-L2 gates
# ---------------------------------------------------------------------------

U32 = 2.0 ** -24
U_OUT = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# smallest positive magnitude of each output type (absolute floor of its rounding)
TINY_OUT = {"f32": 2.0 ** -149, "f16": 2.0 ** -24, "bf16": 2.0 ** -133}


def gamma(n):
    """Worst-case relative error factor of n fp32 roundings in sequence."""
    return n * U32 / (1.0 - n * U32)


def assert_elementwise(y, ref, bound, out_dtype, label=""):
    """|y - ref| <= bound (of the fp32 result) plus the output type's own rounding."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    u = U_OUT[out_dtype]
    lim = (1.0 + u) * bound + u * np.abs(ref) + TINY_OUT[out_dtype]
    bad = ~(np.abs(y - ref) <= lim)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} elements outside the bound, first at {tuple(i)}: "
                             f"got {y[tuple(i)]!r} want {ref[tuple(i)]!r} bound {lim[tuple(i)]!r}")


def column_chunks(N, chunk=8192):
    for c0 in range(0, N, chunk):
        yield np.arange(c0, min(N, c0 + chunk))


def nbits_reference(O, p, A=None, bias=None, bias_dtype="f32", a_mirror=None, w_mirror=None, chunk=8192):
    """Whole-width oracle of a MatMulNBits problem, dequantized one column chunk at a time.

    Returns a dict: "exact" (A . W^T + bias), "mirrored" (with the declared operand
    roundings, when a_mirror / w_mirror are given), "absdot" = sum_k |a'||w'| (rounded
    operands when mirrored), "zsdot" = sum_k |a| |zp * s| and "wsum" = sum_k |w|
    (for the GEMV bound)."""
    A = p["A"] if A is None else A
    a = O.activations_f64(A, p["a_dtype"])
    am = O._round_operand(a, a_mirror) if a_mirror else a
    K, block, bits, N = p["K"], p["block"], p["bits"], p["N"]
    kind = {"packed8": O.ZP_PACKED, "packed": O.ZP_PACKED, "f16_uniform": O.ZP_F16, "f16": O.ZP_F16,
            "none": O.ZP_NONE}[p["zp_mode"]]
    b = None if bias is None else O.activations_f64(bias, bias_dtype)
    out = {k: np.zeros((a.shape[0], N)) for k in ("exact", "absdot", "zsdot")}
    out["wsum"] = np.zeros(N)
    if a_mirror or w_mirror:
        out["mirrored"] = np.zeros((a.shape[0], N))
    for cols in column_chunks(N, chunk):
        zp = None if p["zp"] is None else np.asarray(p["zp"])[cols]
        w = O.dequant_nbits(np.asarray(p["W"])[cols], bits, K, block, np.asarray(p["scales"])[cols], zp,
                            kind).astype(np.float64)
        bc = None if b is None else b[cols]
        out["exact"][:, cols] = O.matmul_f64(a, w, bc)
        wm = O._round_operand(w, w_mirror) if w_mirror else w
        if "mirrored" in out:
            out["mirrored"][:, cols] = O.matmul_f64(am, wm, bc)
        out["absdot"][:, cols] = np.abs(am) @ np.abs(wm).T
        out["zsdot"][:, cols] = np.abs(a) @ _zs(O, p, cols).T
        out["wsum"][cols] = np.abs(w).sum(axis=1)
    return out


def _zs(O, p, rows):
    """|zp * scale| per (row, k) of a MatMulNBits problem, for the GEMV bound."""
    K, block, bits = p["K"], p["block"], p["bits"]
    nblk = (K + block - 1) // block
    mode = p["zp_mode"]
    if mode in ("packed8", "packed"):
        z = O.zero_points_f64(np.asarray(p["zp"])[rows], O.ZP_PACKED, bits, len(rows), nblk)
    elif mode in ("f16_uniform", "f16"):
        z = O.zero_points_f64(np.asarray(p["zp"])[rows], O.ZP_F16, bits, len(rows), nblk)
    else:
        z = O.zero_points_f64(None, O.ZP_NONE, bits, len(rows), nblk)
    s = O.f16_bits_to_f64(np.asarray(p["scales"])[rows]).reshape(len(rows), nblk)
    blk = np.arange(K) // block
    return np.abs(z * s)[:, blk]
