"""Pins for the shared-KV oracle backward (one tensor as keys and values,
CANN sparse_flash_mla_grad "Formula", sliding-window case):

* central finite differences of L = sum(O * dO) where the forward reads the
  one tensor as both keys and values, so a perturbation moves both roles;
* torch fp64 autograd through the library ``scaled_dot_product_attention``
  with one leaf tensor passed as key and value (sink logit as an extra
  zero-value key);
* a planted mistake -- dK alone, the P^T dO term dropped -- fails the
  finite-difference pin;
* the packed (TND) variant equals the dense one sequence by sequence.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import MaskSpec, allowed_mask, backward_shared_kv, forward

from test_oracle_backward import fd_grad


def rand(rng, *shape):
    return rng.standard_normal(shape)


def loss_shared(q, kv, do, scale, spec, sinks):
    o, _ = forward(q, kv, kv, scale, spec, None, sinks)
    return float((o * do).sum())


CASES = [
    # B, Hq, Hk, Sq, Sk, D, spec, sinks
    (1, 2, 1, 5, 6, 3, MaskSpec("none"), False),
    (1, 4, 1, 6, 9, 4, MaskSpec("bottom_right", window_left=3), True),
    (2, 4, 2, 7, 7, 3, MaskSpec("top_left", window_left=2, num_sink=2), True),
    (1, 3, 1, 5, 8, 2, MaskSpec("bottom_right", window_left=2, window_right=1, num_sink=1), False),
]


@pytest.mark.parametrize("case", CASES)
def test_shared_kv_matches_finite_differences(case):
    B, Hq, Hk, Sq, Sk, D, spec, use_sinks = case
    rng = np.random.default_rng(31)
    q, kv, do = rand(rng, B, Hq, Sq, D), rand(rng, B, Hk, Sk, D), rand(rng, B, Hq, Sq, D)
    sinks = rand(rng, Hq) if use_sinks else None
    scale = 0.6
    o, lse = forward(q, kv, kv, scale, spec, None, sinks)
    g = backward_shared_kv(q, kv, o, do, lse, scale, spec, sinks, row_block=4)
    f = lambda: loss_shared(q, kv, do, scale, spec, sinks)  # noqa: E731
    for name, x in [("dq", q), ("dkv", kv)] + ([("dsinks", sinks)] if use_sinks else []):
        ref = fd_grad(x, f)
        np.testing.assert_allclose(g[name], ref, rtol=0, atol=1e-8 * max(1.0, np.abs(ref).max()), err_msg=name)


@pytest.mark.parametrize("case", [
    (2, 8, 1, 40, 64, 32, MaskSpec("bottom_right", window_left=15), True),
    (1, 4, 2, 33, 47, 16, MaskSpec("none"), False),
    (1, 8, 1, 64, 96, 64, MaskSpec("top_left", window_left=20, num_sink=4), True),
])
def test_shared_kv_matches_torch_autograd(case):
    B, Hq, Hk, Sq, Sk, D, spec, use_sinks = case
    rng = np.random.default_rng(32)
    q, kv, do = rand(rng, B, Hq, Sq, D), rand(rng, B, Hk, Sk, D), rand(rng, B, Hq, Sq, D)
    sinks = rand(rng, Hq) if use_sinks else None
    scale = 1.0 / np.sqrt(D)
    o, lse = forward(q, kv, kv, scale, spec, None, sinks)
    g = backward_shared_kv(q, kv, o, do, lse, scale, spec, sinks)

    allowed = allowed_mask(np.arange(Sq)[:, None], np.arange(Sk)[None, :], Sq, Sk, spec)
    qt = torch.tensor(q, requires_grad=True)
    kvt = torch.tensor(kv, requires_grad=True)
    st = torch.tensor(sinks if sinks is not None else np.zeros(Hq), requires_grad=True)
    add = torch.where(torch.from_numpy(allowed), torch.tensor(0.0, dtype=torch.float64),
                      torch.tensor(-np.inf, dtype=torch.float64))[None, None].expand(B, Hq, Sq, Sk)
    kk = vv = kvt
    if sinks is not None:
        kk = torch.cat([kvt, torch.zeros(B, Hk, 1, D, dtype=torch.float64)], dim=2)
        vv = kk
        add = torch.cat([add, st[None, :, None, None].expand(B, Hq, Sq, 1)], dim=3)
    out = F.scaled_dot_product_attention(qt, kk, vv, attn_mask=add, scale=scale, enable_gqa=True)
    (out * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(g["dq"], qt.grad.numpy(), rtol=0, atol=1e-10 * np.abs(g["dq"]).max())
    np.testing.assert_allclose(g["dkv"], kvt.grad.numpy(), rtol=0, atol=1e-10 * np.abs(g["dkv"]).max())
    if sinks is not None:
        np.testing.assert_allclose(g["dsinks"], st.grad.numpy(), rtol=0, atol=1e-10 * np.abs(g["dsinks"]).max())


def test_planted_dk_only_is_caught():
    """dK alone (the P^T dO term of dKV dropped) must fail the FD pin."""
    rng = np.random.default_rng(33)
    q, kv, do = rand(rng, 1, 2, 5, 3), rand(rng, 1, 1, 6, 3), rand(rng, 1, 2, 5, 3)
    spec, scale = MaskSpec("bottom_right", window_left=3), 0.6
    o, lse = forward(q, kv, kv, scale, spec)
    g = oracle.backward(q, kv, kv, o, do, lse, scale, spec)
    ref = fd_grad(kv, lambda: loss_shared(q, kv, do, scale, spec, None))
    assert np.abs(g["dk"] - ref).max() > 1e-3 * np.abs(ref).max()
    assert np.abs(g["dk"] + g["dv"] - ref).max() < 1e-8 * max(1.0, np.abs(ref).max())


def test_shared_kv_varlen_equals_dense_per_sequence():
    rng = np.random.default_rng(34)
    Hq, Hk, D = 4, 1, 8
    lens = [(7, 12), (0, 5), (9, 9)]
    cu_q = np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)
    q, do = rand(rng, int(cu_q[-1]), Hq, D), rand(rng, int(cu_q[-1]), Hq, D)
    kv = rand(rng, int(cu_k[-1]), Hk, D)
    sinks = rand(rng, Hq)
    spec, scale = MaskSpec("bottom_right", window_left=4), 0.5
    max_q = max(a for a, _ in lens)
    o, lse = oracle.forward_varlen(q, kv, kv, cu_q, cu_k, max_q, scale, spec, sinks)
    g = oracle.backward_shared_kv_varlen(q, kv, o, do, lse, cu_q, cu_k, scale, spec, sinks)
    dsinks = np.zeros(Hq)
    for b, (nq, nk) in enumerate(lens):
        q0, k0 = cu_q[b], cu_k[b]
        un = lambda x, a, n: x[a:a + n].transpose(1, 0, 2)[None]  # noqa: E731
        if nq == 0:
            assert np.abs(g["dkv"][k0:k0 + nk]).max() == 0.0
            continue
        od, ld = forward(un(q, q0, nq), un(kv, k0, nk), un(kv, k0, nk), scale, spec, None, sinks)
        gd = backward_shared_kv(un(q, q0, nq), un(kv, k0, nk), od, un(do, q0, nq), ld, scale, spec, sinks)
        np.testing.assert_allclose(g["dq"][q0:q0 + nq], gd["dq"][0].transpose(1, 0, 2), rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["dkv"][k0:k0 + nk], gd["dkv"][0].transpose(1, 0, 2), rtol=0, atol=1e-12)
        dsinks += gd["dsinks"]
    np.testing.assert_allclose(g["dsinks"], dsinks, rtol=0, atol=1e-12)
