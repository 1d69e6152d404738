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
