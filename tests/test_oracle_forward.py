"""Pins for the oracle forward (O, LSE).

* torch fp64 ``scaled_dot_product_attention`` on the CPU (a library routine)
  for every mask kind, bias and GQA ratio; a sink logit enters the library as
  one extra key with a zero value row whose additive mask entry is the sink.
* closed forms: Q = 0 gives uniform attention (O = mean of the allowed value
  rows, LSE = log(n_allowed), plus e^{sink} in the sum with a sink);
  Sk = 1 gives O = V and LSE = the single logit.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import MaskSpec, allowed_mask, forward


def sdpa(q, k, v, scale, spec, bias=None, sinks=None):
    B, Hq, Sq, _ = q.shape
    Hk, Sk = k.shape[1], k.shape[2]
    allowed = allowed_mask(np.arange(Sq)[:, None], np.arange(Sk)[None, :], Sq, Sk, spec)
    add = np.where(allowed, 0.0, -np.inf)[None, None].repeat(Hq, axis=1)
    if bias is not None:
        add = add + bias[None]
    kt, vt = torch.from_numpy(k), torch.from_numpy(v)
    if sinks is not None:
        kt = torch.cat([kt, torch.zeros(B, Hk, 1, k.shape[3], dtype=torch.float64)], dim=2)
        vt = torch.cat([vt, torch.zeros(B, Hk, 1, v.shape[3], dtype=torch.float64)], dim=2)
        col = np.broadcast_to(np.asarray(sinks, np.float64)[None, :, None, None], (1, Hq, Sq, 1))
        add = np.concatenate([add, col], axis=3)
    o = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt,
                                       attn_mask=torch.from_numpy(np.ascontiguousarray(add)),
                                       scale=scale, enable_gqa=True)
    return o.numpy()


def rand(rng, *shape):
    return rng.standard_normal(shape)


CASES = [
    # B, Hq, Hk, Sq, Sk, D, Dv, spec, bias, sinks
    (2, 4, 4, 17, 17, 8, 8, MaskSpec("none"), False, False),
    (1, 8, 2, 33, 33, 16, 8, MaskSpec("top_left"), False, False),
    (2, 4, 1, 20, 31, 8, 12, MaskSpec("bottom_right"), False, False),
    (1, 4, 2, 40, 40, 8, 8, MaskSpec("top_left", window_left=7, num_sink=3), False, False),
    (1, 4, 4, 24, 24, 8, 8, MaskSpec("none"), True, False),
    (1, 8, 1, 30, 30, 8, 8, MaskSpec("top_left", window_left=5, num_sink=2), True, True),
    (2, 6, 3, 19, 25, 4, 4, MaskSpec("bottom_right", window_left=6, window_right=2), False, True),
    (1, 2, 2, 64, 64, 64, 64, MaskSpec("none"), False, False),
]


@pytest.mark.parametrize("case", CASES)
def test_forward_matches_torch_sdpa(case):
    B, Hq, Hk, Sq, Sk, D, Dv, spec, use_bias, use_sinks = case
    rng = np.random.default_rng(7)
    q, k, v = rand(rng, B, Hq, Sq, D), rand(rng, B, Hk, Sk, D), rand(rng, B, Hk, Sk, Dv)
    bias = rand(rng, Hq, Sq, Sk) if use_bias else None
    sinks = rand(rng, Hq) if use_sinks else None
    scale = 1.0 / np.sqrt(D)
    o, lse = forward(q, k, v, scale, spec, bias, sinks, row_block=8)
    ref = sdpa(q, k, v, scale, spec, bias, sinks)
    assert np.isfinite(lse).all()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)


def test_row_block_invariance():
    rng = np.random.default_rng(3)
    q, k, v = rand(rng, 1, 2, 50, 8), rand(rng, 1, 2, 50, 8), rand(rng, 1, 2, 50, 8)
    spec = MaskSpec("top_left", window_left=9, num_sink=2)
    a = forward(q, k, v, 0.3, spec, row_block=7)
    b = forward(q, k, v, 0.3, spec, row_block=512)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a[0], b[0], atol=1e-15)


@pytest.mark.parametrize("spec", [MaskSpec("none"), MaskSpec("top_left"),
                                  MaskSpec("top_left", window_left=4, num_sink=2),
                                  MaskSpec("bottom_right")])
@pytest.mark.parametrize("sink", [None, 0.7])
def test_zero_query_closed_form(spec, sink):
    rng = np.random.default_rng(11)
    Sq, Sk = 13, 16
    q = np.zeros((1, 1, Sq, 4))
    k, v = rand(rng, 1, 1, Sk, 4), rand(rng, 1, 1, Sk, 5)
    sinks = None if sink is None else np.array([sink])
    o, lse = forward(q, k, v, 0.5, spec, sinks=sinks)
    allowed = allowed_mask(np.arange(Sq)[:, None], np.arange(Sk)[None, :], Sq, Sk, spec)
    n = allowed.sum(axis=1)
    den = n + (0.0 if sink is None else np.exp(sink))
    np.testing.assert_allclose(lse[0, 0], np.log(den), rtol=0, atol=1e-14)
    expect = (allowed.astype(float) @ v[0, 0]) / den[:, None]
    np.testing.assert_allclose(o[0, 0], expect, rtol=0, atol=1e-14)


def test_single_key_closed_form():
    rng = np.random.default_rng(5)
    q, k, v = rand(rng, 2, 4, 9, 6), rand(rng, 2, 2, 1, 6), rand(rng, 2, 2, 1, 3)
    o, lse = forward(q, k, v, 0.4, MaskSpec("none"))
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(o[:, h], np.broadcast_to(v[:, g], o[:, h].shape), atol=1e-15)
        np.testing.assert_allclose(lse[:, h], 0.4 * (q[:, h] @ k[:, g, 0][:, :, None])[..., 0], atol=1e-14)


def test_empty_rows():
    """Bottom-right with Sq > Sk leaves the first Sq - Sk rows without keys:
    O = 0 and LSE = -inf there; the other rows are unaffected."""
    rng = np.random.default_rng(9)
    q, k, v = rand(rng, 1, 2, 10, 4), rand(rng, 1, 2, 6, 4), rand(rng, 1, 2, 6, 4)
    o, lse = forward(q, k, v, 0.5, MaskSpec("bottom_right"))
    assert np.isneginf(lse[:, :, :4]).all() and (o[:, :, :4] == 0).all()
    ref = sdpa(q[:, :, 4:], k, v, 0.5, MaskSpec("bottom_right", q_offset=4, sq_total=10, sk_total=6))
    np.testing.assert_allclose(o[:, :, 4:], ref, atol=1e-14)
