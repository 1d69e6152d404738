"""Writes the stored oracle values under tests/golden/ (run from the repository root:
python tests/golden/make_golden.py).

The pages print no input/output values for any of the operations, so these
fixtures are not the pages' numbers: they are the oracle's results on small seeded
problems, frozen so that a later change to the oracle's arithmetic shows up as a
failing test (tests/test_golden.py) and has to be justified by the passage it
follows.  The script calls only the oracle and the seeded input generators.

Definitions followed (by page and section):
  * MatMulNBits, u2/u4 with per-block fp16 scale and zero point:
    hip-ep pull request 1318 "bits=2 MatMulNBits", sections "What" (commit 1) and
    "Performance" (bits=2, block 64, fp16 zero points 1.5, fp32 activations).
  * 16-entry codebook with per-block absmax: bitsandbytes pull request 1979,
    "Technical details".
  * Fused top-k MoE decode fc1 -> SwiGLU -> fc2, fp and int8-activation modes:
    hip-ep pull request 1328, "Summary" and "What".
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from gemm_qmm_nbits_amd import inputs as gen  # noqa: E402
from oracle import qmm_oracle as O  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def hexes(a):
    return [float(v).hex() for v in np.asarray(a, dtype=np.float64).ravel()]


def cases():
    """name -> (description, function returning the fp64 result)."""
    out = {}

    def tiny_u4():
        p = gen.nbits_problem(1, 256, 128, 4, 64, seed=gen.config_seed(0), zp="packed8")
        return O.qmm_nbits(p["A"], "f32", p["W"], 4, 256, 64, p["scales"], p["zp"], O.ZP_PACKED)
    out["tiny_u4_gemv"] = ("tiny u4 GEMV: M=1 K=256 N=128 block 64, packed zero point 8, fp32 A",
                           tiny_u4)

    def u2_uniform_ragged():
        p = gen.nbits_problem(3, 200, 24, 2, 64, seed=77, zp="f16_uniform", uniform_zp=1.5,
                              scale_range=(0.01, 0.05), bias=True)
        return O.qmm_nbits(p["A"], "f32", p["W"], 2, 200, 64, p["scales"], p["zp"], O.ZP_F16,
                           bias=p["bias"])
    out["u2_uniform_zp_ragged"] = ("u2, M=3 K=200 (ragged last block) N=24, block 64, fp16 zero "
                                   "point 1.5 everywhere, fp32 bias", u2_uniform_ragged)

    def codebook():
        p = gen.codebook_problem(2, 128, 16, seed=78, a_dtype="f16")
        return O.qmm_codebook4(p["A"], "f16", p["W"], 128, 64, p["absmax"], p["codebook"])
    out["codebook4_small"] = ("codebook 4-bit, M=2 K=128 N=16, block 64, fp16 A", codebook)

    def moe(mode):
        def f():
            p = gen.qmoe_problem(2, 64, 32, 4, 2, 32, seed=79, zp=True, bias=True)
            return O.qmoe_decode(p["X"], p["ids"], p["rw"], p["fc1"], p["fc2"], 64, 32, 32, mode=mode)
        return f
    out["qmoe_small_fp"] = ("MoE decode fp mode: T=2 H=64 I=32 E=4 k=2 block 32, zero points, bias",
                            moe("fp"))
    out["qmoe_small_int8"] = ("MoE decode int8-activation mode, same problem", moe("int8"))
    return out


def main():
    data = {"note": "oracle results on seeded problems; the pages print no values",
            "cases": {}}
    for name, (desc, f) in cases().items():
        y = f()
        data["cases"][name] = {"description": desc, "shape": list(np.shape(y)), "values_hex": hexes(y)}
    path = os.path.join(HERE, "oracle_small_cases.json")
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
