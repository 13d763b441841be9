"""GPU parity of the shared-KV path: one tensor as keys and values at head
dim 512 (CANN sparse_flash_mla_grad "Formula", sliding-window case), the
HIP library through the C ABI against the fp64 oracle on the same seeded
inputs.

Tolerance: max|gpu - ref| <= 2e-2 * max|ref| (bf16 operands, fp32
accumulation, as for the other bf16 paths), plus an absolute 1e-5 floor.
The backward on both sides consumes the same fp32 O and LSE from the oracle
forward; the GPU forward is checked on its own.
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import MaskSpec
from attention_backward_attn_amd.inputs import SHARED_KV_WORKLOADS, make_shared_kv_inputs, round_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from parity_util import check as _check  # noqa: E402

from attention_backward_attn_amd import binding as ab  # noqa: E402

TOL = 2e-2
D = 512


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    ab.lib()


def dev(x, dtype):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dtype)


def check(name, got, ref, tol=TOL):
    return _check(name, got, ref, tol)


def mask_kw(spec: MaskSpec):
    return dict(mask=spec.kind, window_left=spec.window_left, window_right=spec.window_right,
                num_sink_tokens=spec.num_sink)


def draw(rng, *shape):
    return round_bf16(rng.standard_normal(shape).astype(np.float32))


DENSE = [
    # B, Hq, Hk, Sq, Sk, spec, sinks
    (1, 8, 1, 100, 200, MaskSpec("bottom_right", window_left=63), True),
    (2, 4, 1, 64, 64, MaskSpec("none"), False),
    (1, 4, 2, 130, 130, MaskSpec("top_left", window_left=40, num_sink=4), True),
    (1, 16, 1, 257, 96, MaskSpec("bottom_right"), False),        # rows without keys
    (1, 4, 1, 1, 77, MaskSpec("none"), True),
    (1, 4, 1, 45, 1, MaskSpec("none"), False),
    (1, 64, 1, 96, 320, MaskSpec("bottom_right", window_left=127), True),
]


def dense_inputs(case, seed):
    B, Hq, Hk, Sq, Sk, spec, use_sinks = case
    rng = np.random.default_rng(seed)
    x = {"q": draw(rng, B, Hq, Sq, D), "kv": draw(rng, B, Hk, Sk, D), "do": draw(rng, B, Hq, Sq, D)}
    x["sinks"] = rng.standard_normal(Hq).astype(np.float32) if use_sinks else None
    return x


def case_id(c):
    return f"B{c[0]}H{c[1]}:{c[2]}-S{c[3]}x{c[4]}-{c[5].kind}{c[5].window_left}{'-sinks' if c[6] else ''}"


@pytest.mark.parametrize("case", DENSE, ids=case_id)
def test_forward_parity(case):
    say(f"[shared-kv fwd] {case_id(case)}")
    spec = case[5]
    x = dense_inputs(case, 41)
    scale = 1.0 / np.sqrt(D)
    o_ref, lse_ref = oracle.forward(x["q"], x["kv"], x["kv"], scale, spec, None, x["sinks"])
    q, kv = dev(x["q"], torch.bfloat16), dev(x["kv"], torch.bfloat16)
    o, lse = ab.forward(q, kv, kv, sinks=dev(x["sinks"], torch.float32), scale=scale, **mask_kw(spec))
    torch.cuda.synchronize()
    check("o", o, o_ref)
    lse_g = lse.cpu().numpy()
    empty = np.isneginf(lse_ref)
    assert (np.isneginf(lse_g) == empty).all()
    np.testing.assert_allclose(lse_g[~empty], lse_ref[~empty], rtol=0, atol=1e-3)
    assert (o.cpu()[torch.from_numpy(empty)] == 0).all(), "rows without keys must be zero"


def run_dense_backward(case, seed, flags=0):
    spec = case[5]
    x = dense_inputs(case, seed)
    scale = 1.0 / np.sqrt(D)
    o64, lse64 = oracle.forward(x["q"], x["kv"], x["kv"], scale, spec, None, x["sinks"])
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward_shared_kv(x["q"], x["kv"], o32, x["do"], lse32, scale, spec, x["sinks"])
    q, kv, do = (dev(x[n], torch.bfloat16) for n in ("q", "kv", "do"))
    got = ab.backward(q, kv, kv, dev(o32, torch.float32), do, dev(lse32, torch.float32),
                      sinks=dev(x["sinks"], torch.float32), flags=flags | ab.ATTN_SHARED_KV, scale=scale,
                      **mask_kw(spec))
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("case", DENSE, ids=case_id)
def test_backward_parity(case):
    say(f"[shared-kv bwd] {case_id(case)}")
    got, ref = run_dense_backward(case, 42)
    assert got["dv"] is None
    errs = {"dq": check("dq", got["dq"], ref["dq"]), "dkv": check("dkv", got["dk"], ref["dkv"])}
    if ref["dsinks"] is not None:
        errs["dsinks"] = check("dsinks", got["dsinks"], ref["dsinks"])
    check("delta", got["delta"], ref["delta"], 1e-5)
    say(f"  rel errs {errs}")


def test_deterministic_is_bitwise_repeatable():
    case = DENSE[0]
    say(f"[shared-kv deterministic] {case_id(case)}")
    a, ref = run_dense_backward(case, 43, ab.ATTN_DETERMINISTIC)
    b, _ = run_dense_backward(case, 43, ab.ATTN_DETERMINISTIC)
    assert torch.equal(a["dq"], b["dq"]) and torch.equal(a["dk"], b["dk"])
    check("dkv", a["dk"], ref["dkv"])


@pytest.mark.parametrize("flags", [ab.ATTN_ACCUMULATE_DQ, ab.ATTN_ACCUMULATE_DKDV])
def test_accumulate_into_existing(flags):
    case = DENSE[2]
    say(f"[shared-kv accumulate {flags}] {case_id(case)}")
    spec = case[5]
    x = dense_inputs(case, 44)
    scale = 1.0 / np.sqrt(D)
    o64, lse64 = oracle.forward(x["q"], x["kv"], x["kv"], scale, spec, None, x["sinks"])
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward_shared_kv(x["q"], x["kv"], o32, x["do"], lse32, scale, spec, x["sinks"])
    q, kv, do = (dev(x[n], torch.bfloat16) for n in ("q", "kv", "do"))
    o, lse = dev(o32, torch.float32), dev(lse32, torch.float32)
    rng = np.random.default_rng(45)
    dq0 = rng.standard_normal(x["q"].shape).astype(np.float32)
    dk0 = rng.standard_normal(x["kv"].shape).astype(np.float32)
    dq, dk = dev(dq0, torch.float32), dev(dk0, torch.float32)
    delta = torch.empty(o.shape[:3], device="cuda", dtype=torch.float32)
    p = ab.make_problem(q, kv, kv, o=o, do=do, dq=dq, dk=dk, scale=scale, **mask_kw(spec))
    ab.attn_bwd_preprocess(p, o, do, lse, None, delta, None)
    ab.attn_bwd(p, q, kv, kv, do, lse, delta, None, dq, dk, None, None, flags | ab.ATTN_SHARED_KV)
    torch.cuda.synchronize()
    acc_q = flags & ab.ATTN_ACCUMULATE_DQ
    acc_k = flags & ab.ATTN_ACCUMULATE_DKDV
    check("dq", dq, ref["dq"] + (dq0 if acc_q else 0))
    check("dkv", dk, ref["dkv"] + (dk0 if acc_k else 0))


PACKED = [
    # (query, key) lengths per sequence, Hq, Hk, spec, sinks
    (((37, 90), (0, 20), (64, 64), (100, 50), (5, 0)), 8, 1, MaskSpec("bottom_right", window_left=31), True),
    (((128, 128), (33, 160)), 4, 2, MaskSpec("top_left", window_left=50, num_sink=2), False),
]


@pytest.mark.parametrize("case", PACKED, ids=lambda c: f"n{len(c[0])}-H{c[1]}:{c[2]}-{c[3].kind}")
def test_packed_parity(case):
    seqs, Hq, Hk, spec, use_sinks = case
    say(f"[shared-kv packed] {seqs}")
    cu_q = np.concatenate([[0], np.cumsum([a for a, _ in seqs])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([b for _, b in seqs])]).astype(np.int32)
    max_q, max_k = max(a for a, _ in seqs), max(b for _, b in seqs)
    rng = np.random.default_rng(46)
    x = {"q": draw(rng, int(cu_q[-1]), Hq, D), "kv": draw(rng, int(cu_k[-1]), Hk, D),
         "do": draw(rng, int(cu_q[-1]), Hq, D)}
    sinks = rng.standard_normal(Hq).astype(np.float32) if use_sinks else None
    scale = 1.0 / np.sqrt(D)
    o64, lse64 = oracle.forward_varlen(x["q"], x["kv"], x["kv"], cu_q, cu_k, max_q, scale, spec, sinks)
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward_shared_kv_varlen(x["q"], x["kv"], o32, x["do"], lse32, cu_q, cu_k, scale, spec,
                                           sinks)
    q, kv, do = (dev(x[n], torch.bfloat16) for n in ("q", "kv", "do"))
    kw = dict(cu_seqlens_q=dev(cu_q, torch.int32), cu_seqlens_k=dev(cu_k, torch.int32), max_seqlen_q=max_q,
              max_seqlen_k=max_k, scale=scale, **mask_kw(spec))
    o, lse = ab.forward(q, kv, kv, sinks=dev(sinks, torch.float32), **kw)
    torch.cuda.synchronize()
    check("o", o, o64)
    got = ab.backward(q, kv, kv, dev(o32, torch.float32), do, dev(lse32, torch.float32),
                      sinks=dev(sinks, torch.float32), flags=ab.ATTN_SHARED_KV, **kw)
    torch.cuda.synchronize()
    check("dq", got["dq"], ref["dq"])
    check("dkv", got["dk"], ref["dkv"])
    if sinks is not None:
        check("dsinks", got["dsinks"], ref["dsinks"])


def test_example_size_full_parity():
    """The example's sizes (256 queries, 1024 keys, 64 query heads, one KV
    head, D = 512), every output against the full oracle backward."""
    w = SHARED_KV_WORKLOADS["mla_swa512_s256x1024"]
    say(f"[shared-kv full] {w.name}")
    x = make_shared_kv_inputs(w)
    spec = MaskSpec("bottom_right", window_left=w.window_left)
    o64, lse64 = oracle.forward_varlen(x["q"], x["kv"], x["kv"], x["cu_q"], x["cu_k"], w.max_q, w.scale, spec,
                                       x["sinks"])
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward_shared_kv_varlen(x["q"], x["kv"], o32, x["do"], lse32, x["cu_q"], x["cu_k"], w.scale,
                                           spec, x["sinks"])
    q, kv, do = (dev(x[n], torch.bfloat16) for n in ("q", "kv", "do"))
    kw = dict(cu_seqlens_q=dev(x["cu_q"], torch.int32), cu_seqlens_k=dev(x["cu_k"], torch.int32),
              max_seqlen_q=w.max_q, max_seqlen_k=w.max_k, scale=w.scale, **mask_kw(spec))
    sinks = dev(x["sinks"], torch.float32)
    o, lse = ab.forward(q, kv, kv, sinks=sinks, **kw)
    torch.cuda.synchronize()
    check("o", o, o64)
    got = ab.backward(q, kv, kv, dev(o32, torch.float32), do, dev(lse32, torch.float32), sinks=sinks,
                      flags=ab.ATTN_SHARED_KV, **kw)
    torch.cuda.synchronize()
    errs = {n: check(n, got[g], ref[n]) for n, g in (("dq", "dq"), ("dkv", "dk"), ("dsinks", "dsinks"))}
    say(f"  rel errs {errs}")


def test_long_sequence_sampled():
    """One 4096-token sequence (64 query heads, one KV head, D = 512): the GPU
    forward against the oracle on sampled heads, the GPU backward (on the
    oracle's O / LSE) against the oracle on sampled query rows and keys."""
    w = SHARED_KV_WORKLOADS["mla_swa512_s4096"]
    say(f"[shared-kv sampled] {w.name}")
    x = make_shared_kv_inputs(w)
    spec = MaskSpec("bottom_right", window_left=w.window_left)
    dense = lambda a: a.transpose(1, 0, 2)[None]  # noqa: E731  (one sequence: [1, H, S, D])
    qd, kvd, dod = dense(x["q"]), dense(x["kv"]), dense(x["do"])
    say("  oracle forward (64 heads)")
    o64, lse64 = oracle.forward(qd, kvd, kvd, w.scale, spec, None, x["sinks"], row_block=1024)
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    q, kv, do = (dev(x[n], torch.bfloat16) for n in ("q", "kv", "do"))
    kw = dict(cu_seqlens_q=dev(x["cu_q"], torch.int32), cu_seqlens_k=dev(x["cu_k"], torch.int32),
              max_seqlen_q=w.max_q, max_seqlen_k=w.max_k, scale=w.scale, **mask_kw(spec))
    sinks = dev(x["sinks"], torch.float32)
    say("  GPU forward")
    o, lse = ab.forward(q, kv, kv, sinks=sinks, **kw)
    torch.cuda.synchronize()
    for h in (0, 31, 63):
        check(f"o[h{h}]", o[:, h], o64[0, h])
    say("  GPU backward")
    o_packed = dev(o32[0].transpose(1, 0, 2), torch.float32)
    got = ab.backward(q, kv, kv, o_packed, do, dev(lse32, torch.float32), sinks=sinks, flags=ab.ATTN_SHARED_KV,
                      **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(got["dq"]).all() and torch.isfinite(got["dk"]).all()
    rng = np.random.default_rng(78)
    S = w.max_k
    keys = np.unique(np.concatenate([[0, 1, 2, 511, 512, S // 2, S - 2, S - 1], rng.choice(S, 40, replace=False)]))
    dk_ref, dv_ref = oracle.dkdv_keys(qd, kvd, kvd, o32, dod, lse32, w.scale, spec, 0, 0, keys)
    errs = {"dkv": check("dkv", got["dk"][keys, 0], dk_ref + dv_ref)}
    for h in (0, 17, 63):
        rows = np.unique(np.concatenate([[0, 1, S - 1], rng.choice(S, 32, replace=False)]))
        ref = oracle.dq_rows(qd, kvd, kvd, o32, dod, lse32, w.scale, spec, 0, h, rows)
        errs[f"dq[h{h}]"] = check("dq", got["dq"][rows, h], ref)
    ref_d, ref_s = oracle.preprocess(o32, dod, lse32, x["sinks"])
    errs["dsinks"] = check("dsinks", got["dsinks"], ref_s)
    say(f"  rel errs {errs}")
