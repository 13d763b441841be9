"""Pins for the log-sum-exp merge and the chunked (K/V-split) path.

Ring attention for PyTorch (gist ``ring_attn.py``): ``_ring_fwd`` merges the
partial (o, lse) of each K/V chunk with logaddexp; ``_ring_bwd`` runs the
backward of each chunk against the *global* o and lse and sums dq.  The
merged result must equal the unchunked forward, and the chunked backward
must equal the unchunked backward.
"""
import numpy as np
import pytest

from oracle import MaskSpec, backward, forward, lse_merge


def rand(rng, *shape):
    return rng.standard_normal(shape)


SPECS = [MaskSpec("none"), MaskSpec("top_left"), MaskSpec("bottom_right"),
         MaskSpec("top_left", window_left=10, num_sink=3)]


@pytest.mark.parametrize("spec", SPECS)
@pytest.mark.parametrize("with_sinks", [False, True])
def test_chunked_forward_merge_equals_full(spec, with_sinks):
    rng = np.random.default_rng(3)
    B, Hq, Hk, Sq, Sk, D = 1, 4, 2, 32, 48, 8
    q, k, v = rand(rng, B, Hq, Sq, D), rand(rng, B, Hk, Sk, D), rand(rng, B, Hk, Sk, D)
    sinks = rand(rng, Hq) if with_sinks else None
    o_ref, lse_ref = forward(q, k, v, 0.4, spec, sinks=sinks)
    o = np.zeros((B, Hq, Sq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    n = 4
    c = Sk // n
    for i in range(n):
        sub = MaskSpec(spec.kind, spec.window_left, spec.window_right, spec.num_sink,
                       0, i * c, Sq, Sk)
        # the sink logit joins exactly one chunk's normaliser
        o2, l2 = forward(q, k[:, :, i * c:(i + 1) * c], v[:, :, i * c:(i + 1) * c], 0.4, sub,
                         sinks=sinks if i == 0 else None)
        o, lse = lse_merge(o, lse, o2, l2)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)


def test_merge_identity_and_commutativity():
    rng = np.random.default_rng(4)
    o_a, lse_a = rand(rng, 2, 3, 5, 4), rand(rng, 2, 3, 5)
    o_b, lse_b = rand(rng, 2, 3, 5, 4), rand(rng, 2, 3, 5)
    empty_o, empty_l = np.zeros_like(o_a), np.full_like(lse_a, -np.inf)
    o, l = lse_merge(o_a, lse_a, empty_o, empty_l)
    np.testing.assert_array_equal(l, lse_a)
    np.testing.assert_allclose(o, o_a, atol=1e-15)
    o1, l1 = lse_merge(o_a, lse_a, o_b, lse_b)
    o2, l2 = lse_merge(o_b, lse_b, o_a, lse_a)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(l1, l2, atol=1e-15)
    o, l = lse_merge(empty_o, empty_l, empty_o, empty_l)
    assert np.isneginf(l).all() and (o == 0).all()


def test_merge_weights_closed_form():
    """Two equal partials merge to the same o and lse + log 2."""
    rng = np.random.default_rng(5)
    o_a, lse_a = rand(rng, 1, 2, 6, 3), rand(rng, 1, 2, 6)
    o, l = lse_merge(o_a, lse_a, o_a, lse_a)
    np.testing.assert_allclose(l, lse_a + np.log(2), atol=1e-15)
    np.testing.assert_allclose(o, o_a, atol=1e-15)


@pytest.mark.parametrize("spec", SPECS)
def test_chunked_backward_equals_full(spec):
    rng = np.random.default_rng(6)
    B, Hq, Hk, Sq, Sk, D = 1, 4, 2, 32, 48, 8
    q, k, v, do = rand(rng, B, Hq, Sq, D), rand(rng, B, Hk, Sk, D), rand(rng, B, Hk, Sk, D), rand(rng, B, Hq, Sq, D)
    o, lse = forward(q, k, v, 0.4, spec)
    g = backward(q, k, v, o, do, lse, 0.4, spec)
    dq = np.zeros_like(q)
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    c = Sk // 4
    for i in range(4):
        sub = MaskSpec(spec.kind, spec.window_left, spec.window_right, spec.num_sink, 0, i * c, Sq, Sk)
        gi = backward(q, k[:, :, i * c:(i + 1) * c], v[:, :, i * c:(i + 1) * c], o, do, lse, 0.4, sub)
        dq += gi["dq"]
        dk[:, :, i * c:(i + 1) * c] = gi["dk"]
        dv[:, :, i * c:(i + 1) * c] = gi["dv"]
    np.testing.assert_allclose(dq, g["dq"], atol=1e-13)
    np.testing.assert_allclose(dk, g["dk"], atol=1e-13)
    np.testing.assert_allclose(dv, g["dv"], atol=1e-13)
