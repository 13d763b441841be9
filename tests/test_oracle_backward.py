"""Pins for the oracle backward (dQ, dK, dV, dbias, dsinks) and preprocess.

* central finite differences of L = sum(O * dO) on every element of every
  input -- the verification protocol of CK FMHA example 28 "Backward Bias
  Gradient (dbias) FMHA" (Step 4), here in fp64 over all elements;
* torch fp64 autograd through the library ``scaled_dot_product_attention``
  (bias as an additive float mask with requires_grad; the sink logit as one
  extra zero-value key);
* invariants: per-row sum_j dS = 0 without sinks, hence sum_j dK = 0 and
  sum_j dV = sum_i dO; with sinks the shift invariance
  sum_{b,i,j} dS + dsinks = 0 per head;
* GQA equals MHA on repeated K/V followed by the group sum (example 34
  "Backward Pass with GQA", Step 3);
* Sk = 1: dS = 0, so dQ = dK = 0 and dV = sum of dO over the group.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import MaskSpec, allowed_mask, backward, forward


def rand(rng, *shape):
    return rng.standard_normal(shape)


def loss(q, k, v, do, scale, spec, bias, sinks):
    o, _ = forward(q, k, v, scale, spec, bias, sinks)
    return float((o * do).sum())


def fd_grad(x, f, eps=1e-5):
    g = np.zeros_like(x)
    flat, gf = x.reshape(-1), g.reshape(-1)
    for n in range(flat.size):
        old = flat[n]
        flat[n] = old + eps
        lp = f()
        flat[n] = old - eps
        lm = f()
        flat[n] = old
        gf[n] = (lp - lm) / (2 * eps)
    return g


FD_CASES = [
    # B, Hq, Hk, Sq, Sk, D, Dv, spec, bias, sinks
    (1, 2, 2, 5, 6, 3, 3, MaskSpec("none"), False, False),
    (1, 4, 2, 6, 6, 3, 2, MaskSpec("top_left"), False, False),
    (2, 2, 1, 4, 7, 2, 3, MaskSpec("bottom_right"), True, False),
    (1, 4, 1, 7, 7, 3, 3, MaskSpec("top_left", window_left=2, num_sink=2), False, True),
    (1, 2, 2, 6, 5, 2, 2, MaskSpec("none"), True, True),
    (1, 4, 2, 6, 8, 3, 3, MaskSpec("bottom_right", window_left=3, window_right=1, num_sink=1), True, True),
]


@pytest.mark.parametrize("case", FD_CASES)
def test_backward_matches_finite_differences(case):
    B, Hq, Hk, Sq, Sk, D, Dv, spec, use_bias, use_sinks = case
    rng = np.random.default_rng(21)
    q, k, v = rand(rng, B, Hq, Sq, D), rand(rng, B, Hk, Sk, D), rand(rng, B, Hk, Sk, Dv)
    do = rand(rng, B, Hq, Sq, Dv)
    bias = rand(rng, Hq, Sq, Sk) if use_bias else None
    sinks = rand(rng, Hq) if use_sinks else None
    scale = 0.7
    o, lse = forward(q, k, v, scale, spec, bias, sinks)
    g = backward(q, k, v, o, do, lse, scale, spec, bias, sinks, row_block=3)
    f = lambda: loss(q, k, v, do, scale, spec, bias, sinks)  # noqa: E731
    tol = 1e-8
    for name, x in [("dq", q), ("dk", k), ("dv", v)] + \
            ([("dbias", bias)] if use_bias else []) + ([("dsinks", sinks)] if use_sinks else []):
        ref = fd_grad(x, f)
        np.testing.assert_allclose(g[name], ref, rtol=0, atol=tol * max(1.0, np.abs(ref).max()),
                                   err_msg=name)


def sdpa_autograd(q, k, v, do, scale, spec, bias=None, sinks=None):
    B, Hq, Sq, _ = q.shape
    Hk, Sk = k.shape[1], k.shape[2]
    allowed = allowed_mask(np.arange(Sq)[:, None], np.arange(Sk)[None, :], Sq, Sk, spec)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    bt = torch.tensor(bias if bias is not None else np.zeros((Hq, Sq, Sk)), requires_grad=True)
    st = torch.tensor(sinks if sinks is not None else np.zeros(Hq), requires_grad=True)
    add = torch.where(torch.from_numpy(allowed), bt, torch.tensor(-np.inf, dtype=torch.float64))
    add = add[None].expand(B, Hq, Sq, Sk)
    kk, vv = kt, vt
    if sinks is not None:
        kk = torch.cat([kt, torch.zeros(B, Hk, 1, k.shape[3], dtype=torch.float64)], dim=2)
        vv = torch.cat([vt, torch.zeros(B, Hk, 1, v.shape[3], dtype=torch.float64)], dim=2)
        add = torch.cat([add, st[None, :, None, None].expand(B, Hq, Sq, 1)], dim=3)
    o = F.scaled_dot_product_attention(qt, kk, vv, attn_mask=add, scale=scale, enable_gqa=True)
    (o * torch.from_numpy(do)).sum().backward()
    grad = lambda t: None if t.grad is None else t.grad.numpy()  # noqa: E731
    return {"dq": grad(qt), "dk": grad(kt), "dv": grad(vt), "dbias": grad(bt), "dsinks": grad(st)}


AG_CASES = [
    (2, 8, 2, 40, 40, 16, 16, MaskSpec("top_left"), False, False),
    (1, 4, 4, 33, 47, 8, 12, MaskSpec("bottom_right"), True, False),
    (2, 8, 1, 64, 64, 16, 16, MaskSpec("top_left", window_left=11, num_sink=4), False, True),
    (3, 4, 2, 30, 30, 8, 8, MaskSpec("none"), True, True),
    (1, 2, 2, 64, 64, 64, 64, MaskSpec("none"), False, False),
]


@pytest.mark.parametrize("case", AG_CASES)
def test_backward_matches_torch_autograd(case):
    B, Hq, Hk, Sq, Sk, D, Dv, spec, use_bias, use_sinks = case
    rng = np.random.default_rng(5)
    q, k, v = rand(rng, B, Hq, Sq, D), rand(rng, B, Hk, Sk, D), rand(rng, B, Hk, Sk, Dv)
    do = rand(rng, B, Hq, Sq, Dv)
    bias = rand(rng, Hq, Sq, Sk) if use_bias else None
    sinks = rand(rng, Hq) if use_sinks else None
    scale = 1 / np.sqrt(D)
    o, lse = forward(q, k, v, scale, spec, bias, sinks)
    g = backward(q, k, v, o, do, lse, scale, spec, bias, sinks, row_block=16)
    ref = sdpa_autograd(q, k, v, do, scale, spec, bias, sinks)
    for name in ["dq", "dk", "dv"] + (["dbias"] if use_bias else []) + (["dsinks"] if use_sinks else []):
        np.testing.assert_allclose(g[name], ref[name], rtol=0, atol=1e-12 * max(1, np.abs(ref[name]).max()),
                                   err_msg=name)


def test_invariants_without_sinks():
    rng = np.random.default_rng(8)
    B, Hq, Hk, S, D = 2, 4, 2, 48, 8
    q, k, v, do = rand(rng, B, Hq, S, D), rand(rng, B, Hk, S, D), rand(rng, B, Hk, S, D), rand(rng, B, Hq, S, D)
    bias = rand(rng, Hq, S, S)
    spec = MaskSpec("top_left", window_left=13, num_sink=2)
    o, lse = forward(q, k, v, 0.35, spec, bias)
    g = backward(q, k, v, o, do, lse, 0.35, spec, bias)
    # dbias for B batches is sum_b dS; its rows sum to zero
    np.testing.assert_allclose(g["dbias"].sum(axis=2), 0, atol=1e-13)
    np.testing.assert_allclose(g["dk"].sum(axis=2), 0, atol=1e-13)
    dv_expect = do.reshape(B, Hk, Hq // Hk, S, D).sum(axis=(2, 3))
    np.testing.assert_allclose(g["dv"].sum(axis=2), dv_expect, atol=1e-12)


def test_sink_shift_invariance():
    """Adding c to every logit of a head and to its sink leaves O unchanged,
    so sum_{b,i,j} dS + dsinks = 0 for that head."""
    rng = np.random.default_rng(13)
    B, Hq, Hk, S, D = 2, 4, 1, 40, 8
    q, k, v, do = rand(rng, B, Hq, S, D), rand(rng, B, Hk, S, D), rand(rng, B, Hk, S, D), rand(rng, B, Hq, S, D)
    bias = np.zeros((Hq, S, S))
    sinks = rand(rng, Hq)
    spec = MaskSpec("top_left", window_left=7, num_sink=3)
    o, lse = forward(q, k, v, 0.35, spec, bias, sinks)
    g = backward(q, k, v, o, do, lse, 0.35, spec, bias, sinks)
    np.testing.assert_allclose(g["dbias"].sum(axis=(1, 2)) + g["dsinks"], 0, atol=1e-12)


def test_gqa_equals_expanded_mha():
    rng = np.random.default_rng(2)
    B, Hq, Hk, S, D = 2, 8, 2, 24, 8
    G = Hq // Hk
    q, k, v, do = rand(rng, B, Hq, S, D), rand(rng, B, Hk, S, D), rand(rng, B, Hk, S, D), rand(rng, B, Hq, S, D)
    spec = MaskSpec("top_left")
    o, lse = forward(q, k, v, 0.3, spec)
    g = backward(q, k, v, o, do, lse, 0.3, spec)
    ke, ve = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    oe, lsee = forward(q, ke, ve, 0.3, spec)
    np.testing.assert_allclose(oe, o, atol=1e-15)
    ge = backward(q, ke, ve, oe, do, lsee, 0.3, spec)
    np.testing.assert_allclose(ge["dq"], g["dq"], atol=1e-14)
    np.testing.assert_allclose(ge["dk"].reshape(B, Hk, G, S, D).sum(axis=2), g["dk"], atol=1e-13)
    np.testing.assert_allclose(ge["dv"].reshape(B, Hk, G, S, D).sum(axis=2), g["dv"], atol=1e-13)


def test_single_key_gradients():
    rng = np.random.default_rng(4)
    q, k, v, do = rand(rng, 1, 4, 9, 5), rand(rng, 1, 2, 1, 5), rand(rng, 1, 2, 1, 6), rand(rng, 1, 4, 9, 6)
    o, lse = forward(q, k, v, 0.5, MaskSpec("none"))
    g = backward(q, k, v, o, do, lse, 0.5, MaskSpec("none"))
    assert np.abs(g["dq"]).max() < 1e-14 and np.abs(g["dk"]).max() < 1e-14
    np.testing.assert_allclose(g["dv"][0, :, 0], do[0].reshape(2, 2, 9, 6).sum(axis=(1, 2)), atol=1e-14)


def test_empty_rows_have_zero_gradients():
    rng = np.random.default_rng(6)
    q, k, v, do = rand(rng, 1, 2, 10, 4), rand(rng, 1, 2, 6, 4), rand(rng, 1, 2, 6, 4), rand(rng, 1, 2, 10, 4)
    spec = MaskSpec("bottom_right")
    o, lse = forward(q, k, v, 0.5, spec)
    g = backward(q, k, v, o, do, lse, 0.5, spec)
    assert (g["dq"][:, :, :4] == 0).all()
    # the remaining rows give the same dK/dV as the problem without them
    sub = MaskSpec("bottom_right", q_offset=4, sq_total=10, sk_total=6)
    g2 = backward(q[:, :, 4:], k, v, o[:, :, 4:], do[:, :, 4:], lse[:, :, 4:], 0.5, sub)
    np.testing.assert_allclose(g["dk"], g2["dk"], atol=1e-14)
    np.testing.assert_allclose(g["dv"], g2["dv"], atol=1e-14)


def test_sampled_helpers_match_full_backward():
    rng = np.random.default_rng(10)
    B, Hq, Hk, S, D = 2, 4, 2, 40, 8
    q, k, v, do = rand(rng, B, Hq, S, D), rand(rng, B, Hk, S, D), rand(rng, B, Hk, S, D), rand(rng, B, Hq, S, D)
    bias = rand(rng, Hq, S, S)
    spec = MaskSpec("top_left", window_left=9, num_sink=2)
    o, lse = forward(q, k, v, 0.3, spec, bias)
    g = backward(q, k, v, o, do, lse, 0.3, spec, bias)
    rows = np.array([0, 3, 17, 39])
    np.testing.assert_allclose(oracle.dq_rows(q, k, v, o, do, lse, 0.3, spec, 1, 3, rows, bias),
                               g["dq"][1, 3, rows], atol=1e-13)
    keys = np.array([0, 1, 2, 20, 39])
    dk, dv = oracle.dkdv_keys(q, k, v, o, do, lse, 0.3, spec, 0, 1, keys, bias)
    np.testing.assert_allclose(dk, g["dk"][0, 1, keys], atol=1e-13)
    np.testing.assert_allclose(dv, g["dv"][0, 1, keys], atol=1e-13)
    dbias_rows = sum(oracle.ds_rows(q, k, v, o, do, lse, 0.3, spec, bb, 2, rows, bias) for bb in range(B))
    np.testing.assert_allclose(dbias_rows, g["dbias"][2, rows], atol=1e-13)


def test_planted_mistake_is_caught():
    """A plausible oracle mistake (dropping the D term of dS) must fail the
    finite-difference pin: the pin is not vacuous."""
    rng = np.random.default_rng(1)
    q, k, v, do = rand(rng, 1, 2, 5, 3), rand(rng, 1, 2, 5, 3), rand(rng, 1, 2, 5, 3), rand(rng, 1, 2, 5, 3)
    o, lse = forward(q, k, v, 0.5, MaskSpec("none"))
    wrong = backward(q, k, v, np.zeros_like(o), do, lse, 0.5, MaskSpec("none"))  # D = 0
    ref = fd_grad(q, lambda: loss(q, k, v, do, 0.5, MaskSpec("none"), None, None))
    assert np.abs(wrong["dq"] - ref).max() > 1e-3
