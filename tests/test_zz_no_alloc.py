"""attn_bwd_static (the entry point that allocates nothing, its partial sums
in the library's static device scratch) against attn_bwd with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
problem, each starting from NaN-filled outputs.  Both entry points run the
same kernels and sum the split parts in the same slot order, so the results
agree bit for bit (and hence within the parity bound)."""

import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from attention_backward_attn_amd import binding as ab  # noqa: E402
from parity_util import TOL, check  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(B, Hq, Hk, S, D, mask, seed, window_left=-1, num_sink=0, sinks=False):
    g = torch.Generator().manual_seed(seed)
    q, do = (torch.randn(B, Hq, S, D, generator=g).to("cuda", torch.bfloat16) for _ in range(2))
    k, v = (torch.randn(B, Hk, S, D, generator=g).to("cuda", torch.bfloat16) for _ in range(2))
    sk = torch.randn(Hq, generator=g).to("cuda") if sinks else None
    kw = dict(mask=mask, window_left=window_left, num_sink_tokens=num_sink)
    o, lse = ab.forward(q, k, v, sinks=sk, scale=D ** -0.5, **kw)
    dq, dk, dv = (torch.empty(t.shape, device="cuda") for t in (q, k, v))
    delta = torch.empty_like(lse)
    dsinks = torch.empty(Hq, device="cuda") if sinks else None
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, scale=D ** -0.5, **kw)
    ab.attn_bwd_preprocess(p, o, do, lse, sk, delta, dsinks, None, None, None)
    return p, (q, k, v, do, lse, delta), (dq, dk, dv)


@pytest.mark.parametrize("flags", [0, ab.ATTN_DETERMINISTIC], ids=["default", "determ"])
def test_static_scratch_matches_workspace(flags):
    cases = [
        # the small GQA workload's shape: key blocks split eight ways (56 MiB of partial sums)
        dict(B=2, Hq=16, Hk=4, S=1024, D=128, mask="top_left", seed=1),
        # smaller, and a sliding window with sink tokens (the sink block's parts only)
        dict(B=1, Hq=16, Hk=2, S=640, D=128, mask="top_left", seed=2, window_left=127, num_sink=4, sinks=True),
    ]
    for c in cases:
        say(f"[no alloc] {c} flags={flags}")
        p, (q, k, v, do, lse, delta), (dq, dk, dv) = _case(**c)
        need = ab.attn_bwd_workspace_size(p, flags)
        assert 0 < need <= ab.ATTN_STATIC_SCRATCH_BYTES, need
        ws = ab.set_workspace(p, flags)
        ab.attn_bwd(p, q, k, v, do, lse, delta, None, dq, dk, dv, None, flags)
        torch.cuda.synchronize()
        ref = [t.clone() for t in (dq, dk, dv)]
        del ws
        p.workspace, p.workspace_bytes = None, 0
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        ab.attn_bwd_static(p, q, k, v, do, lse, delta, None, dq, dk, dv, None, flags)
        torch.cuda.synchronize()
        for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            check(name, got, r.cpu().numpy(), TOL["bf16"])
            assert torch.equal(got, r), name


def test_static_scratch_rejects_oversized():
    """A problem whose partial sums exceed the static scratch is refused
    with ATTN_ENOSCRATCH, before any kernel runs: the outputs keep their
    contents."""
    B, Hq, Hk, S, D = 1, 8, 1, 12288, 128   # key blocks split eight ways: 84 MiB of partial sums
    q = torch.empty(B, Hq, S, D, device="cuda", dtype=torch.bfloat16)
    k = torch.empty(B, Hk, S, D, device="cuda", dtype=torch.bfloat16)
    o = torch.empty(B, Hq, S, D, device="cuda")
    dq, dk = torch.full(q.shape, 7.0, device="cuda"), torch.full(k.shape, 7.0, device="cuda")
    lse = torch.empty(B, Hq, S, device="cuda")
    p = ab.make_problem(q, k, k, o=o, do=q, dq=dq, dk=dk, dv=dk, mask="top_left")
    assert ab.attn_bwd_workspace_size(p) > ab.ATTN_STATIC_SCRATCH_BYTES
    with pytest.raises(ab.AttnError) as e:
        ab.attn_bwd_static(p, q, k, k, q, lse, lse, None, dq, dk, dk, None, 0)
    assert e.value.status == ab.ATTN_ENOSCRATCH
    torch.cuda.synchronize()
    assert (dq == 7.0).all() and (dk == 7.0).all()
