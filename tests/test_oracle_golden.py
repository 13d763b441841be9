"""Regression pin: the oracle still reproduces the stored fixtures in
tests/golden/ (written by tests/golden/make_golden.py from the oracle after
it passed its finite-difference and library pins).  A change to the oracle's
arithmetic shows up here first."""
import json
import os
import sys

import numpy as np
import pytest

from oracle import MaskSpec, backward, forward

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, HERE)
import make_golden  # noqa: E402


@pytest.mark.parametrize("name", sorted(make_golden.CASES))
def test_golden(name):
    with open(os.path.join(HERE, name + ".json")) as f:
        ref = json.load(f)
    c = ref["case"]
    q, k, v, do, bias, sinks = make_golden.build(c)
    spec = MaskSpec(**c["spec"])
    o, lse = forward(q, k, v, c["scale"], spec, bias, sinks)
    g = backward(q, k, v, o, do, lse, c["scale"], spec, bias, sinks)
    np.testing.assert_allclose(o, ref["o"], atol=1e-14)
    np.testing.assert_allclose(lse, ref["lse"], atol=1e-14)
    for key in ("dq", "dk", "dv", "dbias", "dsinks"):
        if ref[key] is None:
            assert g[key] is None
        else:
            np.testing.assert_allclose(g[key], ref[key], atol=1e-13, err_msg=key)
