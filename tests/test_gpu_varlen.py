"""GPU parity of the variable-length packed batch (TND tensors with
cumulative sequence lengths, [SFMG] "Prototype") against the varlen oracle,
through the C ABI: forward (O, LSE) and backward (dQ, dK, dV, delta,
dsinks), ragged lengths including empty sequences and q / k lengths that
differ per sequence."""

import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import MaskSpec
from attention_backward_attn_amd.inputs import round_bf16

pytestmark = pytest.mark.gpu

from parity_util import check as _check  # noqa: E402

from attention_backward_attn_amd import binding as ab  # noqa: E402

TOL = 2e-2      # bf16 matrix-core operands, fp32 accumulation


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    ab.lib()


def check(name, got, ref, tol):
    return _check(name, got, ref, tol)


CASES = [
    # cu_q, cu_k, Hq, Hk, D, spec, sinks
    ([0, 100, 100, 357, 620], [0, 100, 100, 357, 620], 8, 2, 128, MaskSpec("bottom_right"), False),
    ([0, 33, 290, 291, 700], [0, 150, 170, 300, 800], 4, 4, 128, MaskSpec("bottom_right"), False),
    ([0, 64, 64, 513], [0, 64, 80, 600], 8, 1, 64, MaskSpec("top_left", window_left=40, num_sink=3), True),
    ([0, 200, 201, 460], [0, 129, 390, 391], 4, 2, 128, MaskSpec("none"), True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
@pytest.mark.parametrize("flags", [0, ab.ATTN_DETERMINISTIC], ids=["default", "determ"])
def test_varlen_parity(case, flags):
    cu_q, cu_k, Hq, Hk, D, spec, with_sinks = case
    say(f"[varlen] {case} flags={flags}")
    cu_q, cu_k = np.array(cu_q), np.array(cu_k)
    max_q = int(np.diff(cu_q).max())
    max_k = int(np.diff(cu_k).max())
    rng = np.random.default_rng(int(cu_q[-1] + cu_k[-1]))
    f = lambda *s: round_bf16(rng.standard_normal(s).astype(np.float32))
    q, k, v, do = f(cu_q[-1], Hq, D), f(cu_k[-1], Hk, D), f(cu_k[-1], Hk, D), f(cu_q[-1], Hq, D)
    sinks = rng.standard_normal(Hq).astype(np.float32) if with_sinks else None
    scale = 1 / np.sqrt(D)
    o64, lse64 = oracle.forward_varlen(q, k, v, cu_q, cu_k, max_q, scale, spec, sinks)

    dev = lambda a, t: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda", t)
    qd, kd, vd, dod = (dev(a, torch.bfloat16) for a in (q, k, v, do))
    sd = dev(sinks, torch.float32)
    cq, ck = dev(cu_q.astype(np.int32), torch.int32), dev(cu_k.astype(np.int32), torch.int32)
    kw = dict(mask=spec.kind, window_left=spec.window_left, window_right=spec.window_right,
              num_sink_tokens=spec.num_sink, cu_seqlens_q=cq, cu_seqlens_k=ck, max_seqlen_q=max_q,
              max_seqlen_k=max_k)
    # forward
    o, lse = ab.forward(qd, kd, vd, sinks=sd, scale=scale, **kw)
    torch.cuda.synchronize()
    check("o", o, o64, TOL)
    lse_g = lse.cpu().numpy()
    for b in range(len(cu_q) - 1):
        n = cu_q[b + 1] - cu_q[b]
        ref = lse64[b, :, :n]
        assert (np.isneginf(lse_g[b, :, :n]) == np.isneginf(ref)).all()
        fin = np.isfinite(ref)
        np.testing.assert_allclose(lse_g[b, :, :n][fin], ref[fin], rtol=0, atol=1e-4)
    # backward on the oracle's O / LSE (fp32)
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward_varlen(q, k, v, o32, do, lse32, cu_q, cu_k, scale, spec, sinks)
    got = ab.backward(qd, kd, vd, dev(o32, torch.float32), dod, dev(lse32, torch.float32), sinks=sd,
                      flags=flags, scale=scale, **kw)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv"):
        check(n, got[n], ref[n], TOL)
    if with_sinks:
        check("dsinks", got["dsinks"], ref["dsinks"], TOL)
    d = got["delta"].cpu().numpy()
    for b in range(len(cu_q) - 1):
        n = cu_q[b + 1] - cu_q[b]
        np.testing.assert_allclose(d[b, :, :n], ref["delta"][b, :, :n], rtol=1e-5, atol=1e-5)
        assert np.all(d[b, :, n:] == 0), "delta past a sequence's length must be 0"


def test_varlen_rejects_bias_and_fp32():
    cu = torch.tensor([0, 8, 16], dtype=torch.int32, device="cuda")
    q = torch.zeros(16, 2, 64, dtype=torch.bfloat16, device="cuda")
    kw = dict(cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=8, max_seqlen_k=8)
    bias = torch.zeros(2, 8, 8, device="cuda")
    with pytest.raises(ab.AttnError) as e:
        ab.forward(q, q, q, bias=bias, **kw)
    assert e.value.status == ab.ATTN_EUNSUPPORTED
    qf = q.float()
    with pytest.raises(ab.AttnError) as e:
        ab.forward(qf, qf, qf, **kw)
    assert e.value.status == ab.ATTN_EUNSUPPORTED
