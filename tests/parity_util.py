"""Shared tolerance check of the GPU parity tests, with a record of every
achieved margin.

The bound per output tensor is  max|gpu - ref| <= tol * max|ref|  with
tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (fp32 accumulation).
There is no absolute term, except for a reference that is identically zero
in exact arithmetic (max|ref| below ZERO_REF: e.g. dQ and dK when every row
has a single key, where dS = P (dP - delta) vanishes and the fp64 oracle
leaves rounding noise of ~1e-17).  Such an output must stay below ZERO_ATOL
in absolute terms: fp32 rounding of delta = rowsum(dO * O) against
dP = dO V^T leaves ~1e-7 * |dO| |V| behind on the GPU.

Every check appends (test, output, max|err| / max|ref|, tol) to MARGINS;
tests/conftest.py prints the table at the end of the session, so a run's
log shows how far inside the bound each output landed.
"""

from __future__ import annotations

import os

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}
ZERO_REF = 1e-6
ZERO_ATOL = 1e-5

MARGINS: list = []


def _current_test() -> str:
    t = os.environ.get("PYTEST_CURRENT_TEST", "?")
    return t.split(" ")[0].split("::")[-1]


def to_f64(x) -> np.ndarray:
    try:
        import torch
        if torch.is_tensor(x):
            return x.detach().float().cpu().numpy().astype(np.float64)
    except ImportError:
        pass
    return np.asarray(x, dtype=np.float64)


def check(name: str, got, ref, tol: float) -> float:
    """Assert the bound above for one output; returns max|err| / max|ref|
    (or max|err| for an essentially zero reference)."""
    got = to_f64(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    if ref.size == 0:
        return 0.0
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    if scale < ZERO_REF:
        MARGINS.append((_current_test(), name, err, ZERO_ATOL, "abs"))
        assert err <= ZERO_ATOL, f"{name}: zero reference, max |gpu| {err:.3e} > {ZERO_ATOL:g}"
        return err
    rel = err / scale
    MARGINS.append((_current_test(), name, rel, tol, "rel"))
    assert err <= tol * scale, f"{name}: max err {err:.3e} > {tol:g} * {scale:.3e} (rel {rel:.3e})"
    return rel
