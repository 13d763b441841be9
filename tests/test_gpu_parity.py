"""GPU parity: the HIP library (through the C ABI) against the fp64 CPU oracle
on the same seeded inputs.

Tolerance (per output tensor): max|gpu - ref| <= tol * max|ref|, with
tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (fp32 accumulation).
There is no absolute term except for references that are zero in exact
arithmetic (see parity_util).  The backward on both sides consumes the same
fp32 O and LSE, produced by the oracle forward, so parity measures the
backward kernels alone; the GPU forward is checked separately.  The three
large workloads (headline, ALiBi + dbias, window + sink) and the 4-chunk
headline are compared element by element on every output, with oracle
references computed over (batch entry, KV head) units in a forked worker
pool (oracle_pool).
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import MaskSpec
from attention_backward_attn_amd.inputs import WORKLOADS, make_inputs, round_bf16
from parity_util import TOL, check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from attention_backward_attn_amd import binding as ab  # noqa: E402



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


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def mask_kw(spec: MaskSpec):
    return dict(mask=spec.kind, window_left=spec.window_left, window_right=spec.window_right,
                num_sink_tokens=spec.num_sink, q_offset=spec.q_offset, k_offset=spec.k_offset,
                sq_total=spec.sq_total or 0, sk_total=spec.sk_total or 0)


def random_case(B, Hq, Hk, Sq, Sk, D, Dv, dtype, seed, bias, sinks):
    rng = np.random.default_rng(seed)
    f = (lambda a: round_bf16(a.astype(np.float32))) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    x = {"q": f(rng.standard_normal((B, Hq, Sq, D))), "k": f(rng.standard_normal((B, Hk, Sk, D))),
         "v": f(rng.standard_normal((B, Hk, Sk, Dv))), "do": f(rng.standard_normal((B, Hq, Sq, Dv)))}
    x["bias"] = rng.standard_normal((Hq, Sq, Sk)).astype(np.float32) if bias else None
    x["sinks"] = rng.standard_normal(Hq).astype(np.float32) if sinks else None
    return x


def run_full_parity(x, dtype, spec, scale, flags=0, workspace=True):
    """Oracle forward -> fp32 O/LSE -> GPU and oracle backward; compare all."""
    o64, lse64 = oracle.forward(x["q"], x["k"], x["v"], scale, spec, x["bias"], x["sinks"])
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward(x["q"], x["k"], x["v"], o32, x["do"], lse32, scale, spec, x["bias"], x["sinks"])
    dt = tdtype(dtype)
    q, k, v, do = (dev(x[n], dt) for n in ("q", "k", "v", "do"))
    bias, sinks = dev(x["bias"], torch.float32), dev(x["sinks"], torch.float32)
    o, lse = dev(o32, torch.float32), dev(lse32, torch.float32)
    got = ab.backward(q, k, v, o, do, lse, bias=bias, sinks=sinks, want_dbias=bias is not None,
                      flags=flags, scale=scale, workspace=workspace, **mask_kw(spec))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    errs = {}
    for n in ("dq", "dk", "dv", "dbias", "dsinks"):
        if ref[n] is not None:
            errs[n] = check(n, got[n], ref[n], tol)
    check("delta", got["delta"], ref["delta"], 1e-5)
    return errs, got


SMALL = [
    # B, Hq, Hk, Sq, Sk, D, Dv, dtype, spec, bias, sinks
    (1, 2, 2, 64, 64, 64, 64, "f32", MaskSpec("none"), False, False),
    (2, 4, 2, 77, 77, 64, 64, "f32", MaskSpec("top_left"), True, True),
    (1, 4, 4, 100, 130, 32, 48, "f32", MaskSpec("bottom_right"), False, False),
    (2, 8, 2, 256, 256, 128, 128, "bf16", MaskSpec("top_left"), False, False),
    (1, 8, 1, 300, 300, 128, 128, "bf16", MaskSpec("bottom_right"), False, False),
    (2, 4, 4, 192, 320, 64, 64, "bf16", MaskSpec("none"), True, False),
    (1, 16, 2, 384, 384, 128, 128, "bf16", MaskSpec("top_left", window_left=100, num_sink=4), False, True),
    (1, 4, 1, 200, 333, 128, 128, "bf16", MaskSpec("bottom_right", window_left=63, window_right=5,
                                                    num_sink=3), True, True),
    (2, 2, 1, 257, 129, 64, 64, "bf16", MaskSpec("bottom_right"), False, False),   # empty rows
    (1, 2, 2, 1, 513, 128, 128, "bf16", MaskSpec("none"), False, False),
    (1, 8, 8, 129, 1, 64, 64, "bf16", MaskSpec("none"), False, False),
    (1, 4, 2, 96, 112, 128, 64, "bf16", MaskSpec("top_left"), False, True),      # Dqk != Dv
    (3, 4, 4, 640, 640, 64, 64, "bf16", MaskSpec("none"), True, False),           # batch-ordered dbias
    (1, 32, 8, 1100, 1100, 128, 128, "bf16", MaskSpec("bottom_right"), False, False),
    (1, 16, 1, 512, 512, 64, 64, "bf16", MaskSpec("top_left"), False, False),     # D = 64, 16-way split
    # head dim 64 with a bias and dbias under masks (masked tiles of both passes)
    (2, 4, 2, 200, 333, 64, 64, "bf16", MaskSpec("bottom_right", window_left=63, window_right=5,
                                                  num_sink=3), True, True),
    (5, 2, 2, 160, 160, 64, 64, "bf16", MaskSpec("top_left"), True, False),       # two batch groups
    (1, 4, 4, 256, 200, 64, 64, "bf16", MaskSpec("bottom_right"), True, False),
    # 64-row query tiles of the dK/dV pass: one partial tile with a bias at
    # head dim 64; three tiles with a 2-row tail at head dim 128
    (1, 2, 2, 40, 96, 64, 64, "bf16", MaskSpec("bottom_right"), True, False),
    (2, 4, 1, 130, 70, 128, 128, "bf16", MaskSpec("top_left"), False, True),
    # head dim 64 without a bias on a grid of 512 dQ workgroups (two per CU:
    # the dQ pass with issue priorities)
    (1, 32, 8, 2048, 2048, 64, 64, "bf16", MaskSpec("bottom_right"), False, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[7]}-B{c[0]}H{c[1]}:{c[2]}-S{c[3]}x{c[4]}-D{c[5]}-"
                         f"{c[8].kind}{'-bias' if c[9] else ''}{'-sinks' if c[10] else ''}")
@pytest.mark.parametrize("flags", [0, ab.ATTN_DETERMINISTIC], ids=["atomic", "determ"])
@pytest.mark.parametrize("workspace", [True, False], ids=["ws", "nows"])
def test_small_parity(case, flags, workspace):
    """With a workspace, the parts of split key blocks keep partial dK / dV
    sums that are added in slot order; without one they add atomically into
    zeroed outputs."""
    B, Hq, Hk, Sq, Sk, D, Dv, dtype, spec, bias, sinks = case
    say(f"[parity] {case} flags={flags} workspace={workspace}")
    x = random_case(B, Hq, Hk, Sq, Sk, D, Dv, dtype, 100 + Sq + Sk, bias, sinks)
    run_full_parity(x, dtype, spec, 1.0 / np.sqrt(D), flags, workspace)


@pytest.mark.parametrize("name", ["mha_f32_s64", "gqa4_causal_tl_s1024"])
def test_workload_full_parity(name):
    w = WORKLOADS[name]
    say(f"[workload full] {name}")
    x = make_inputs(w)
    spec = MaskSpec(w.mask, w.window_left, w.window_right, w.num_sink)
    errs, _ = run_full_parity(x, w.dtype, spec, w.scale)
    say(f"  rel errs {errs}")


def gpu_backward_full(w, x, ref, flags=0):
    """GPU preprocess + attn_bwd of workload ``w`` on the oracle's fp32 O / LSE."""
    spec = MaskSpec(w.mask, w.window_left, w.window_right, w.num_sink)
    dt = tdtype(w.dtype)
    q, k, v, do = (dev(x[n], dt) for n in ("q", "k", "v", "do"))
    bias, sinks = dev(x["bias"], torch.float32), dev(x["sinks"], torch.float32)
    o, lse = dev(ref["o"], torch.float32), dev(ref["lse"], torch.float32)
    say(f"[full] {w.name}: GPU backward flags={flags}")
    got = ab.backward(q, k, v, o, do, lse, bias=bias, sinks=sinks, want_dbias=bias is not None,
                      flags=flags, scale=w.scale, **mask_kw(spec))
    torch.cuda.synchronize()
    return got, (q, k, v, do, bias, sinks, o, lse)


def compare_full(w, got, ref):
    tol = TOL[w.dtype]
    errs = {}
    for n in ("dq", "dk", "dv", "dbias", "dsinks"):
        if ref[n] is not None:
            errs[n] = check(n, got[n], ref[n], tol)
    check("delta", got["delta"], ref["delta"], 1e-5)
    say(f"  rel errs {errs}")
    return errs


def full_workload(name):
    """Full-size run of a workload, every element of every output compared
    with the oracle: the GPU forward (O, LSE) against the oracle forward,
    and the GPU backward on the oracle's fp32 O / LSE against the oracle
    backward (dQ, dK, dV, dbias over all [Hq, Sq, Sk], dsinks over all Hq,
    delta)."""
    import oracle_pool
    w = WORKLOADS[name]
    x = make_inputs(w)
    spec = MaskSpec(w.mask, w.window_left, w.window_right, w.num_sink)
    say(f"[full] {name}: oracle references")
    ref = oracle_pool.reference(name, w, x, spec, say)
    got, t = gpu_backward_full(w, x, ref)
    compare_full(w, got, ref)
    del got
    q, k, v, do, bias, sinks, _, _ = t
    say(f"[full] {name}: GPU forward")
    o_g, lse_g = ab.forward(q, k, v, bias=bias, sinks=sinks, scale=w.scale, **mask_kw(spec))
    torch.cuda.synchronize()
    lse_g = lse_g.cpu().numpy()
    assert not np.isneginf(ref["lse"]).any() and np.isfinite(lse_g).all()
    check("lse", lse_g, ref["lse"], 1e-5)
    check("o", o_g, ref["o64"], TOL[w.dtype])
    return w, x, ref


@pytest.mark.full_oracle
@pytest.mark.timeout(900)
def test_headline_full():
    full_workload("gqa4_causal_br_s4096")


@pytest.mark.full_oracle
@pytest.mark.timeout(900)
def test_alibi_dbias_full():
    import oracle_pool
    full_workload("mha_alibi_dbias_s2048")
    oracle_pool.drop("mha_alibi_dbias_s2048")


@pytest.mark.full_oracle
@pytest.mark.timeout(1200)
def test_window_sink_full():
    import oracle_pool
    full_workload("gqa8_swa1024_sink4_s8192")
    oracle_pool.drop("gqa8_swa1024_sink4_s8192")


def test_dsinks_full_batch():
    """dsinks sums over the batch: check it on a small multi-batch case."""
    x = random_case(3, 8, 2, 160, 160, 64, 64, "bf16", 5, False, True)
    run_full_parity(x, "bf16", MaskSpec("top_left", window_left=31, num_sink=2), 0.125)


# ---------------------------------------------------------------------------
FWD = [
    (1, 2, 2, 64, 64, 64, 64, "f32", MaskSpec("none"), False, False),
    (2, 8, 2, 200, 200, 128, 128, "bf16", MaskSpec("top_left", window_left=50, num_sink=3), True, True),
    (1, 4, 1, 100, 260, 128, 64, "bf16", MaskSpec("bottom_right"), False, True),    # Dqk != Dv
    (1, 2, 2, 90, 40, 64, 64, "bf16", MaskSpec("bottom_right"), False, False),       # empty rows
    (1, 8, 2, 1100, 1100, 128, 128, "bf16", MaskSpec("bottom_right"), False, False),
    (2, 4, 4, 300, 260, 64, 64, "bf16", MaskSpec("none"), True, False),
    (1, 4, 2, 333, 333, 64, 64, "bf16", MaskSpec("top_left", window_left=40, num_sink=2), False, True),
    (1, 4, 1, 130, 700, 128, 128, "bf16", MaskSpec("bottom_right", window_left=63, window_right=5,
                                                    num_sink=3), True, True),
    (1, 2, 2, 50, 1, 128, 128, "bf16", MaskSpec("none"), False, False),              # one key
    (1, 2, 1, 70, 20, 64, 64, "bf16", MaskSpec("top_left", window_left=3), False, False),  # empty rows, window
]


def fwd_case(case, o_dtype=None):
    B, Hq, Hk, Sq, Sk, D, Dv, dtype, spec, bias, sinks = case
    x = random_case(B, Hq, Hk, Sq, Sk, D, Dv, dtype, 3, bias, sinks)
    o_ref, lse_ref = oracle.forward(x["q"], x["k"], x["v"], 1 / np.sqrt(D), spec, x["bias"], x["sinks"])
    dt = tdtype(dtype)
    o, lse = ab.forward(dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt), bias=dev(x["bias"], torch.float32),
                        sinks=dev(x["sinks"], torch.float32), scale=1 / np.sqrt(D), o_dtype=o_dtype,
                        **mask_kw(spec))
    torch.cuda.synchronize()
    lse_g = lse.cpu().numpy()
    empty = np.isneginf(lse_ref)
    assert (np.isneginf(lse_g) == empty).all()
    np.testing.assert_allclose(lse_g[~empty], lse_ref[~empty], rtol=0, atol=1e-4)
    assert (o.cpu()[torch.from_numpy(empty)] == 0).all(), "rows without keys must be zero"
    return o, o_ref


@pytest.mark.parametrize("case", FWD)
def test_forward_parity(case):
    say(f"[fwd] {case}")
    o, o_ref = fwd_case(case)
    # bf16 inputs: P is a bf16 matrix-core operand
    check("o", o, o_ref, 1e-4 if case[7] == "f32" else TOL["bf16"])


def test_forward_bf16_output():
    case = FWD[4]
    say(f"[fwd bf16 O] {case}")
    o, o_ref = fwd_case(case, o_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    check("o", o, o_ref, TOL["bf16"])


# (B, Hq, Hk, S, D, dtype, mask, bias): the matrix-core path (head dims 128
# and 64 with a bias) and the fp32 path
BSHD_CASES = [(2, 8, 2, 200, 128, "bf16", MaskSpec("bottom_right"), False),
              (2, 4, 4, 160, 64, "bf16", MaskSpec("top_left"), True),
              (1, 4, 2, 96, 64, "f32", MaskSpec("none"), False)]


def bshd_view(a, dtype):
    """numpy [B, H, S, D] -> device memory in [B, S, H, D] order, returned as
    its [B, H, S, D] view (row stride H D, head stride D)."""
    t = torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3))).to("cuda", dtype)
    return t.transpose(1, 2)


@pytest.mark.parametrize("case", BSHD_CASES, ids=["gqa_d128", "bias_d64", "f32"])
def test_bshd_layout(case):
    """Tensors stored [B, S, H, D] (native BSHD, the Ascend interface's
    layout option) pass through the ABI as strides: the forward O and every
    gradient match the oracle as for [B, H, S, D] storage."""
    B, Hq, Hk, S, D, dtype, spec, with_bias = case
    say(f"[bshd] {case}")
    x = random_case(B, Hq, Hk, S, S, D, D, dtype, 41, with_bias, False)
    scale = 1 / np.sqrt(D)
    o64, lse64 = oracle.forward(x["q"], x["k"], x["v"], scale, spec, x["bias"])
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward(x["q"], x["k"], x["v"], o32, x["do"], lse32, scale, spec, x["bias"])
    dt = tdtype(dtype)
    q, k, v, do = (bshd_view(x[n], dt) for n in ("q", "k", "v", "do"))
    nan = lambda a: bshd_view(np.full(a.shape, np.nan, np.float32), torch.float32)
    o = nan(o32)
    lse = torch.empty(B, Hq, S, device="cuda")
    dq, dk, dv = nan(ref["dq"]), nan(ref["dk"]), nan(ref["dv"])
    bias = dev(x["bias"], torch.float32)
    dbias = None if bias is None else torch.full_like(bias, float("nan"))
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, bias=bias, scale=scale, **mask_kw(spec))
    assert tuple(p.q_str) == (S * Hq * D, D, Hq * D)
    ab.attn_fwd_lse(p, q, k, v, bias, None, o, lse)
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == "f32" else TOL["bf16"]
    check("o", o.cpu().numpy().astype(np.float64), o64, tol)
    # the backward from the oracle's O / LSE, O stored [B, S, H, D] too
    o_in, lse_in = bshd_view(o32, torch.float32), dev(lse32, torch.float32)
    delta = torch.empty_like(lse_in)
    ab.attn_bwd_preprocess(p, o_in, do, lse_in, None, delta, None, None, None, None)
    ab.attn_bwd(p, q, k, v, do, lse_in, delta, bias, dq, dk, dv, dbias, 0)
    torch.cuda.synchronize()
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dbias", dbias)):
        if t is not None:
            check(n, t.cpu().numpy().astype(np.float64), ref[n], tol)


def test_lse_merge_parity():
    say("[merge]")
    rng = np.random.default_rng(12)
    B, H, S, Dv = 2, 3, 70, 96
    o_a, o_b = rng.standard_normal((B, H, S, Dv)).astype(np.float32), rng.standard_normal((B, H, S, Dv)).astype(np.float32)
    l_a, l_b = rng.standard_normal((B, H, S)).astype(np.float32), rng.standard_normal((B, H, S)).astype(np.float32)
    l_a[0, 0, :5] = -np.inf
    o_a[0, 0, :5] = 0
    l_b[0, 0, 3:8] = -np.inf
    o_b[0, 0, 3:8] = 0
    o_ref, l_ref = oracle.lse_merge(o_a, l_a, o_b, l_b)
    oa, la = dev(o_a, torch.float32), dev(l_a, torch.float32)
    ab.attn_lse_merge(oa, la, dev(o_b, torch.float32), dev(l_b, torch.float32))
    torch.cuda.synchronize()
    check("o", oa, o_ref, 1e-6)
    lg = la.cpu().numpy()
    assert (np.isneginf(lg) == np.isneginf(l_ref)).all()
    fin = np.isfinite(l_ref)
    np.testing.assert_allclose(lg[fin], l_ref[fin], atol=1e-6)


@pytest.mark.full_oracle
@pytest.mark.timeout(900)
def test_headline_chunked():
    """The headline workload run as 4 K/V chunks of 1024 ("Ring attention for
    PyTorch", _ring_fwd / _ring_bwd on one GPU): forward partials joined by
    attn_lse_merge, compared with the oracle forward in full; then the
    backward of each chunk against the global O / LSE / delta (the oracle's
    fp32 O / LSE) with dQ accumulated over the chunks and each chunk's dK /
    dV written into its slice, compared in full with the oracle backward."""
    import oracle_pool
    w = WORKLOADS["gqa4_causal_br_s4096"]
    x = make_inputs(w)
    spec = MaskSpec(w.mask)
    ref = oracle_pool.reference(w.name, w, x, spec, say)
    dt = torch.bfloat16
    q, k, v, do = (dev(x[n], dt) for n in ("q", "k", "v", "do"))
    say("[chunked] forward")
    n, c = w.kv_chunks, w.Sk // w.kv_chunks
    o = torch.zeros(w.B, w.Hq, w.Sq, w.Dv, device="cuda")
    lse = torch.full((w.B, w.Hq, w.Sq), -np.inf, device="cuda")
    for i in range(n):
        kc, vc = k[:, :, i * c:(i + 1) * c], v[:, :, i * c:(i + 1) * c]
        o2, l2 = ab.forward(q, kc, vc, scale=w.scale, mask=w.mask, k_offset=i * c, sk_total=w.Sk)
        ab.attn_lse_merge(o, lse, o2, l2)
    torch.cuda.synchronize()
    assert (lse == -np.inf).sum() == 0
    check("o merged", o, ref["o64"], TOL["bf16"])
    check("lse merged", lse, ref["lse"], 1e-5)
    say("[chunked] backward")
    o, lse = dev(ref["o"], torch.float32), dev(ref["lse"], torch.float32)
    dq = torch.full((w.B, w.Hq, w.Sq, w.Dqk), float("nan"), device="cuda")
    dk = torch.full((w.B, w.Hk, w.Sk, w.Dqk), float("nan"), device="cuda")
    dv = torch.full((w.B, w.Hk, w.Sk, w.Dv), float("nan"), device="cuda")
    delta = torch.empty(w.B, w.Hq, w.Sq, device="cuda")
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, scale=w.scale, mask=w.mask)
    # delta only: the first chunk writes every dQ row (over the NaNs), the
    # others add to it -- the page's zeroed dq plus each chunk's share
    ab.attn_bwd_preprocess(p, o, do, lse, None, delta, None, None, None, None)
    keep = []
    for i in range(n):
        sl = slice(i * c, (i + 1) * c)
        pc = ab.make_problem(q, k[:, :, sl], v[:, :, sl], o=o, do=do, dq=dq, dk=dk[:, :, sl], dv=dv[:, :, sl],
                             scale=w.scale, mask=w.mask, k_offset=i * c, sk_total=w.Sk)
        fl = ab.ATTN_ACCUMULATE_DQ if i > 0 else 0
        keep.append(ab.set_workspace(pc, fl))
        ab.attn_bwd(pc, q, k[:, :, sl], v[:, :, sl], do, lse, delta, None, dq, dk[:, :, sl], dv[:, :, sl],
                    None, fl)
    torch.cuda.synchronize()
    del keep
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        check(f"chunked {name}", t, ref[name], TOL["bf16"])
    check("delta", delta, ref["delta"], 1e-5)


@pytest.mark.parametrize("D", [128, 64])
def test_deterministic_is_bitwise_repeatable(D):
    x = random_case(5 if D == 64 else 1, 8, 2, 512, 512, D, D, "bf16", 9, True, True)
    spec = MaskSpec("top_left", window_left=200, num_sink=4)
    dt = torch.bfloat16
    q, k, v, do = (dev(x[n], dt) for n in ("q", "k", "v", "do"))
    bias, sinks = dev(x["bias"], torch.float32), dev(x["sinks"], torch.float32)
    o, lse = ab.forward(q, k, v, bias=bias, sinks=sinks, scale=1 / np.sqrt(D), **mask_kw(spec))
    outs = []
    for _ in range(3):
        g = ab.backward(q, k, v, o, do, lse, bias=bias, sinks=sinks, want_dbias=True,
                        flags=ab.ATTN_DETERMINISTIC, scale=1 / np.sqrt(D), **mask_kw(spec))
        torch.cuda.synchronize()
        outs.append({kk: vv.clone() for kk, vv in g.items() if vv is not None})
    for kk in outs[0]:
        assert torch.equal(outs[0][kk], outs[1][kk]) and torch.equal(outs[0][kk], outs[2][kk]), kk


# (B, Hq, Hk, S, D, bias): no bias (k_dkdv3 / k_dq2); a bias with dbias at
# head dim 64 (k_dkdv3 with the bias, k_dqb) and at head dim 128 (k_dkdv
# walking the batch, k_dq with the bias)
ACC_CASES = [(1, 8, 2, 300, 128, False), (2, 4, 4, 200, 64, True), (2, 2, 2, 160, 128, True)]


@pytest.mark.parametrize("case", ACC_CASES, ids=["nobias", "bias_d64", "bias_d128"])
@pytest.mark.parametrize("flags", [0, ab.ATTN_DETERMINISTIC], ids=["atomic", "determ"])
def test_accumulate_into_existing(flags, case):
    """ATTN_ACCUMULATE_DQ / ATTN_ACCUMULATE_DKDV add into the caller's
    buffers: start from random contents and compare with contents + oracle
    (dbias, when asked, is written, not added)."""
    B, Hq, Hk, S, D, with_bias = case
    x = random_case(B, Hq, Hk, S, S, D, D, "bf16", 21, with_bias, False)
    spec = MaskSpec("top_left")
    scale = 1 / np.sqrt(D)
    say(f"[accumulate] case={case} flags={flags}")
    o64, lse64 = oracle.forward(x["q"], x["k"], x["v"], scale, spec, x["bias"])
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward(x["q"], x["k"], x["v"], o32, x["do"], lse32, scale, spec, x["bias"])
    dt = torch.bfloat16
    q, k, v, do = (dev(x[n], dt) for n in ("q", "k", "v", "do"))
    o, lse = dev(o32, torch.float32), dev(lse32, torch.float32)
    bias = dev(x["bias"], torch.float32)
    dbias = None if bias is None else torch.full_like(bias, float("nan"))
    rng = np.random.default_rng(3)
    init = {n: rng.standard_normal(ref[n].shape).astype(np.float32) for n in ("dq", "dk", "dv")}
    dq, dk, dv = (dev(init[n], torch.float32) for n in ("dq", "dk", "dv"))
    delta = torch.empty_like(lse)
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, bias=bias, scale=scale, mask="top_left")
    ab.attn_bwd_preprocess(p, o, do, lse, None, delta, None, None, None, None)
    ab.attn_bwd(p, q, k, v, do, lse, delta, bias, dq, dk, dv, dbias,
                flags | ab.ATTN_ACCUMULATE_DQ | ab.ATTN_ACCUMULATE_DKDV)
    torch.cuda.synchronize()
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        got = t.cpu().numpy().astype(np.float64) - init[n]
        check(n, got, ref[n], 2e-2)
    if dbias is not None:
        check("dbias", dbias.cpu().numpy().astype(np.float64), ref["dbias"], 2e-2)


@pytest.mark.parametrize("shape", [(1, 4, 1, 200, 700), (4, 8, 8, 256, 2048)], ids=["split", "unsplit"])
@pytest.mark.parametrize("flags", [0, ab.ATTN_DETERMINISTIC], ids=["atomic", "determ"])
def test_unseen_keys_overwritten(shape, flags):
    """Keys that no query row sees (top-left mask with Sk > Sq) get zero
    dK / dV, and every other output its oracle value, when the output
    buffers start out holding NaN: no row of dQ / dK / dV is left unwritten,
    whether the key blocks are split over workgroups or not."""
    B, Hq, Hk, Sq, Sk = shape
    D = 128
    say(f"[unseen keys] {shape} flags={flags}")
    x = random_case(B, Hq, Hk, Sq, Sk, D, D, "bf16", 31, False, False)
    spec = MaskSpec("top_left")
    scale = 1 / np.sqrt(D)
    o64, lse64 = oracle.forward(x["q"], x["k"], x["v"], scale, spec)
    o32, lse32 = o64.astype(np.float32), lse64.astype(np.float32)
    ref = oracle.backward(x["q"], x["k"], x["v"], o32, x["do"], lse32, scale, spec)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    o, lse = dev(o32, torch.float32), dev(lse32, torch.float32)
    dq, dk, dv = (torch.full(t.shape, float("nan"), device="cuda") for t in (q, k, v))
    delta = torch.empty_like(lse)
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, scale=scale, mask="top_left")
    ab.attn_bwd_preprocess(p, o, do, lse, None, delta, None, None, None, None)
    for use_ws in (False, True):   # split parts adding atomically, then keeping partial sums
        ws = ab.set_workspace(p, flags) if use_ws else None  # noqa: F841
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        ab.attn_bwd(p, q, k, v, do, lse, delta, None, dq, dk, dv, None, flags)
        torch.cuda.synchronize()
        for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            check(f"{n} (workspace {use_ws})", t, ref[n], 2e-2)
        assert (dk[:, :, Sq:] == 0).all() and (dv[:, :, Sq:] == 0).all()


def test_split_units_bitwise_repeatable():
    """Without a bias the key-block parts of a split unit leave partial sums
    that are added in a fixed order: repeated calls agree bit for bit, with
    or without ATTN_DETERMINISTIC (the small GQA workload splits each unit
    eight ways)."""
    w = WORKLOADS["gqa4_causal_tl_s1024"]
    x = make_inputs(w)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    o, lse = ab.forward(q, k, v, scale=w.scale, mask=w.mask)
    outs = []
    for flags in (0, 0, ab.ATTN_DETERMINISTIC):
        g = ab.backward(q, k, v, o, do, lse, flags=flags, scale=w.scale, mask=w.mask)
        torch.cuda.synchronize()
        outs.append({n: g[n].clone() for n in ("dq", "dk", "dv")})
    for n in ("dq", "dk", "dv"):
        assert torch.equal(outs[0][n], outs[1][n]) and torch.equal(outs[0][n], outs[2][n]), n


@pytest.mark.parametrize("name", ["gqa4_causal_tl_s1024", "gqa4_causal_br_s4096"])
def test_graph_capture_replays(name):
    """attn_bwd_preprocess + attn_bwd captured into a HIP graph: every
    replay, with eager calls and synchronizations between the replays,
    reproduces the eager result bit for bit (no memset nodes and no
    allocation inside the capture; the small workload sums its eight parts
    per key block in slot order through the caller's workspace, the
    headline adds its two parts atomically onto zero)."""
    w = WORKLOADS[name]
    say(f"[graph] {name}")
    x = make_inputs(w)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    o, lse = ab.forward(q, k, v, scale=w.scale, mask=w.mask)
    dq, dk, dv = (torch.empty(t.shape, device="cuda") for t in (q, k, v))
    delta = torch.empty_like(lse)
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, scale=w.scale, mask=w.mask)
    ws = ab.set_workspace(p)  # noqa: F841

    def step(st):
        ab.attn_bwd_preprocess(p, o, do, lse, None, delta, None, None, None, None, st)
        ab.attn_bwd(p, q, k, v, do, lse, delta, None, dq, dk, dv, None, 0, st)

    main = torch.cuda.current_stream()
    step(main)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i in range(3):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(a, b), f"replay {i}: {n}"
        step(main)   # eager work between the replays
        torch.cuda.synchronize()


def test_no_query_rows_split_parts():
    """No query rows (Sq = 0) with 64 query heads on one KV head: the key
    blocks still split into eight parts, every part stores zeros, and with no
    dQ pass to follow, a kernel of its own sums the partial slots: dK and dV
    (NaN-filled before) come out zero."""
    B, Hq, Hk, Sk, D = 1, 64, 1, 512, 128
    say("[no rows] Sq=0, Hq=64, Hk=1, Sk=512")
    g = torch.Generator().manual_seed(5)
    k, v = (torch.randn(B, Hk, Sk, D, generator=g).to("cuda", torch.bfloat16) for _ in range(2))
    q = torch.empty(B, Hq, 0, D, device="cuda", dtype=torch.bfloat16)
    do = torch.empty_like(q)
    o = torch.empty(B, Hq, 0, D, device="cuda")
    lse = torch.empty(B, Hq, 0, device="cuda")
    delta = torch.empty_like(lse)
    dq = torch.empty(B, Hq, 0, D, device="cuda")
    dk, dv = (torch.full(t.shape, float("nan"), device="cuda") for t in (k, v))
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, scale=D ** -0.5, mask="none")
    ws = ab.set_workspace(p)
    assert ws is not None   # the eight parts keep partial sums
    ab.attn_bwd(p, q, k, v, do, lse, delta, None, dq, dk, dv, None, 0)
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()



@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("with_sinks", [False, True], ids=["nosinks", "sinks"])
def test_no_keys_and_empty_batch(dtype, D, with_sinks):
    """No keys (Sk = 0): every row's O is 0 and its LSE is -inf, or the sink
    logit when the head has one (the oracle's values); the backward gives
    dQ = 0 (NaN-filled before), delta = 0 and dsinks = 0.  An empty batch
    (B = 0) runs the forward and the backward without error."""
    say(f"[no keys] {dtype} D={D} sinks={with_sinks}")
    dt = tdtype(dtype)
    x = random_case(2, 4, 2, 70, 0, D, D, dtype, 21, False, with_sinks)
    spec = MaskSpec("top_left")
    o64, lse64 = oracle.forward(x["q"], x["k"], x["v"], D ** -0.5, spec, None, x["sinks"])
    q, k, v, do = (dev(x[n], dt) for n in ("q", "k", "v", "do"))
    sinks = dev(x["sinks"], torch.float32)
    o, lse = ab.forward(q, k, v, sinks=sinks, **mask_kw(spec))
    torch.cuda.synchronize()
    assert (o == 0).all()
    lse_g, lse_r = lse.cpu().numpy(), lse64.astype(np.float32)
    assert (np.isneginf(lse_g) == np.isneginf(lse_r)).all()
    fin = ~np.isneginf(lse_r)
    np.testing.assert_allclose(lse_g[fin], lse_r[fin], rtol=0, atol=1e-5)
    dq = torch.full(q.shape, float("nan"), device="cuda")
    got = ab.backward(q, k, v, o, do, lse, sinks=sinks, dq=dq, **mask_kw(spec))
    torch.cuda.synchronize()
    assert (got["dq"] == 0).all() and (got["delta"] == 0).all()
    if with_sinks:
        assert (got["dsinks"] == 0).all()
    # empty batch
    e = random_case(0, 4, 2, 70, 50, D, D, dtype, 22, False, with_sinks)
    qe, ke, ve, doe = (dev(e[n], dt) for n in ("q", "k", "v", "do"))
    oe, lsee = ab.forward(qe, ke, ve, sinks=sinks, **mask_kw(spec))
    ge = ab.backward(qe, ke, ve, oe, doe, lsee, sinks=sinks, **mask_kw(spec))
    torch.cuda.synchronize()
    assert ge["dq"].numel() == 0 and ge["dk"].numel() == 0
    if with_sinks:
        assert (ge["dsinks"] == 0).all()

def test_preprocess_zeroes_gradients():
    x = random_case(2, 4, 2, 130, 150, 64, 64, "bf16", 8, False, False)
    dt = torch.bfloat16
    q, k, v, do = (dev(x[n], dt) for n in ("q", "k", "v", "do"))
    o = torch.randn(2, 4, 130, 64, device="cuda")
    lse = torch.randn(2, 4, 130, device="cuda")
    dq = torch.full((2, 4, 130, 64), 7.0, device="cuda")
    dk = torch.full((2, 2, 150, 64), 7.0, device="cuda")
    dv = torch.full((2, 2, 150, 64), 7.0, device="cuda")
    delta = torch.empty_like(lse)
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv)
    ab.attn_bwd_preprocess(p, o, do, lse, None, delta, None, dq, dk, dv)
    torch.cuda.synchronize()
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()
    ref = (do.float() * o).sum(-1)
    assert torch.allclose(delta, ref, atol=1e-4, rtol=1e-5)
