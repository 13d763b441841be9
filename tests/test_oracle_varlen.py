"""Pins of the variable-length packed-batch oracle ([SFMG] "Prototype": TND
layout with cumulative sequence lengths): an equal-length packed batch is the
dense batch; a sequence never sees another's keys; empty sequences give
nothing.  The dense oracle it is built from is pinned in the other files."""

import numpy as np
import pytest

import oracle
from oracle import MaskSpec


def _pack(x):
    """[B, H, S, D] -> packed [B * S, H, D]."""
    B, H, S, D = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B * S, H, D)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("spec", [MaskSpec("none"), MaskSpec("bottom_right"),
                                  MaskSpec("top_left", window_left=3, num_sink=1)])
def test_equal_lengths_match_dense(spec):
    rng = np.random.default_rng(5)
    B, Hq, Hk, S, D = 3, 4, 2, 9, 8
    q, k, v, do = _rand(rng, B, Hq, S, D), _rand(rng, B, Hk, S, D), _rand(rng, B, Hk, S, D), _rand(rng, B, Hq, S, D)
    sinks = _rand(rng, Hq)
    cu = np.arange(B + 1) * S
    o, lse = oracle.forward(q, k, v, 0.3, spec, None, sinks)
    ov, lv = oracle.forward_varlen(_pack(q), _pack(k), _pack(v), cu, cu, S, 0.3, spec, sinks)
    np.testing.assert_allclose(ov, _pack(o), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lv), np.isneginf(lse))
    np.testing.assert_allclose(lv[np.isfinite(lv)], lse[np.isfinite(lse)], rtol=0, atol=1e-13)
    g = oracle.backward(q, k, v, o, do, lse, 0.3, spec, None, sinks)
    gv = oracle.backward_varlen(_pack(q), _pack(k), _pack(v), _pack(o), _pack(do), lse, cu, cu, 0.3, spec, sinks)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(gv[n], _pack(g[n]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(gv["dsinks"], g["dsinks"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(gv["delta"], g["delta"], rtol=0, atol=1e-12)


def test_sequences_are_independent_and_empty_ones_vanish():
    rng = np.random.default_rng(6)
    Hq, Hk, D = 2, 1, 4
    cu_q = np.array([0, 5, 5, 12])     # middle sequence has no rows
    cu_k = np.array([0, 3, 7, 15])     # ... but has keys
    Tq, Tk = cu_q[-1], cu_k[-1]
    q, do = _rand(rng, Tq, Hq, D), _rand(rng, Tq, Hq, D)
    k, v = _rand(rng, Tk, Hk, D), _rand(rng, Tk, Hk, D)
    spec = MaskSpec("bottom_right")
    o, lse = oracle.forward_varlen(q, k, v, cu_q, cu_k, 7, 0.5, spec)
    g = oracle.backward_varlen(q, k, v, o, do, lse, cu_q, cu_k, 0.5, spec)
    # keys of the row-less sequence get no gradient
    assert np.all(g["dk"][3:7] == 0) and np.all(g["dv"][3:7] == 0)
    # the last sequence alone, as a dense problem, gives the same numbers
    sl_q, sl_k = slice(5, 12), slice(7, 15)
    to_d = lambda x: x.transpose(1, 0, 2)[None]
    o3, l3 = oracle.forward(to_d(q[sl_q]), to_d(k[sl_k]), to_d(v[sl_k]), 0.5, spec)
    np.testing.assert_allclose(o[sl_q], o3[0].transpose(1, 0, 2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[2, :, :7], l3[0], rtol=0, atol=1e-13)
    g3 = oracle.backward(to_d(q[sl_q]), to_d(k[sl_k]), to_d(v[sl_k]), o3, to_d(do[sl_q]), l3, 0.5, spec)
    np.testing.assert_allclose(g["dk"][sl_k], g3["dk"][0].transpose(1, 0, 2), rtol=0, atol=1e-12)
    # bottom-right alignment is per sequence: row 0 of the last sequence sees 8 - 7 + 1 = 2 keys
    m = oracle.allowed_mask(np.arange(7)[:, None], np.arange(8)[None, :], 7, 8, spec)
    assert m[0].sum() == 2
    # padded LSE rows stay -inf, padded delta rows 0
    assert np.all(np.isneginf(lse[0, :, 5:])) and np.all(g["delta"][0, :, 5:] == 0)
