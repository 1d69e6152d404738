"""The oracle reproduces its stored values on small seeded problems (tests/golden/).

The pages print no input/output values, so the stored values come from
tests/golden/make_golden.py, which calls only the oracle.  A change to the oracle's
arithmetic fails here and must name the passage that justifies it.  Values are compared
to 1e-10 relative, far below any change of definition and far above fp64 summation-order
differences between BLAS builds.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_reproduces_stored_values():
    with open(os.path.join(HERE, "golden", "oracle_small_cases.json")) as fh:
        data = json.load(fh)
    cases = make_golden.cases()
    assert set(cases) == set(data["cases"])
    for name, (_, f) in cases.items():
        y = np.asarray(f(), dtype=np.float64)
        stored = data["cases"][name]
        assert list(y.shape) == stored["shape"], name
        want = np.array([float.fromhex(v) for v in stored["values_hex"]]).reshape(y.shape)
        # fp64 sums through numpy's BLAS: the order, and so the last bits, may differ
        # between machines; everything else in these cases is exact or rounded once
        assert np.allclose(y, want, rtol=1e-10, atol=1e-13), name
