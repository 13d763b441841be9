"""CPU-side checks of the C ABI: the library loads, exports every entry point
declared in include/*.h, and rejects invalid arguments on the host before any
HIP call (no GPU is touched by these tests)."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

from attention_backward_attn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(attn_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("attn_fwd_lse", "attn_bwd_preprocess", "attn_bwd", "attn_lse_merge"):
        assert n in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports(name):
    L = B.lib()
    assert hasattr(L, name), name
    assert name in B.EXPORTED


def problem(**kw):
    p = B.attn_problem_t()
    B.lib().attn_problem_init(ctypes.byref(p), 1, 4, 2, 64, 64, 64, 64)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_problem_init_defaults():
    p = problem()
    assert abs(p.scale - 0.125) < 1e-7
    assert tuple(p.q_str) == (4 * 64 * 64, 64 * 64, 64)
    assert tuple(p.k_str) == (2 * 64 * 64, 64 * 64, 64)
    assert p.window_left == -1 and p.window_right == 0 and p.mask == 0
    assert tuple(p.bias_str) == (64 * 64, 64)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


BAD = [
    dict(Hk=3),                 # Hq % Hk != 0
    dict(Dqk=0),
    dict(Dv=600),               # above the largest head dim (512)
    dict(scale=0.0),
    dict(scale=float("nan")),
    dict(in_dtype=7),
    dict(mask=5),
    dict(window_left=-2),
    dict(window_right=-1),
    dict(num_sink_tokens=-1),
    dict(window_left=3),        # window with mask NONE
    dict(num_sink_tokens=2),    # sinks with mask NONE
    dict(mask=1, q_offset=10, sq_total=32),   # offset + Sq beyond the global length
    dict(mask=2, k_offset=-1),
    dict(cu_seqlens_q=0x1000),                                  # packed batch needs both prefix sums
    dict(cu_seqlens_q=0x1000, cu_seqlens_k=0x1000, mask=2, sq_total=128),   # no offsets with a packed batch
    dict(cu_seqlens_q=0x1000, cu_seqlens_k=0x1000, total_q=-1),
]


@pytest.mark.parametrize("kw", BAD)
def test_bwd_rejects_invalid_problem(kw):
    p = problem(**kw)
    s = B.lib().attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                         None, 0, None)
    assert s == B.ATTN_EINVAL


@pytest.mark.parametrize("kw", BAD)
def test_fwd_rejects_invalid_problem(kw):
    p = problem(**kw)
    s = B.lib().attn_fwd_lse(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None)
    assert s in (B.ATTN_EINVAL, B.ATTN_EUNSUPPORTED)


def test_packed_batch_unsupported_cases():
    # fp32 inputs and a bias are not covered by the packed-batch kernels;
    # the call fails before any HIP call
    for kw in (dict(in_dtype=0), dict()):
        p = problem(cu_seqlens_q=0x1000, cu_seqlens_k=0x1000, total_q=64, total_k=64, **kw)
        bias = FAKE if not kw else None
        s = B.lib().attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bias, FAKE, FAKE, FAKE,
                             None, 0, None)
        assert s == B.ATTN_EUNSUPPORTED, kw


def test_bwd_rejects_null_pointers_and_flags():
    p = problem()
    L = B.lib()
    assert L.attn_bwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None,
                      0, None) == B.ATTN_EINVAL
    assert L.attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None,
                      0, None) == B.ATTN_EINVAL
    # dbias without bias
    assert L.attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                      0, None) == B.ATTN_EINVAL
    # unknown flag bit
    assert L.attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None,
                      16, None) == B.ATTN_EINVAL
    assert L.attn_bwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, 0,
                      None) == B.ATTN_EINVAL


def test_preprocess_sinks_pairing():
    p = problem()
    L = B.lib()
    # sinks without dsinks and the reverse
    assert L.attn_bwd_preprocess(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None, None) == B.ATTN_EINVAL
    assert L.attn_bwd_preprocess(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, None, None) == B.ATTN_EINVAL


def test_fp32_large_head_dim_unsupported():
    p = problem(in_dtype=B.ATTN_F32, Dqk=192, Dv=192)
    s = B.lib().attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                         None, 0, None)
    assert s == B.ATTN_EUNSUPPORTED


def test_merge_validation_and_empty():
    L = B.lib()
    assert L.attn_lse_merge(1, 1, 4, 0, FAKE, FAKE, FAKE, FAKE, None) == B.ATTN_EINVAL
    assert L.attn_lse_merge(-1, 1, 4, 8, FAKE, FAKE, FAKE, FAKE, None) == B.ATTN_EINVAL
    assert L.attn_lse_merge(1, 1, 4, 8, None, FAKE, FAKE, FAKE, None) == B.ATTN_EINVAL
    # zero rows: nothing to do, no device access
    assert L.attn_lse_merge(0, 4, 4, 8, None, None, None, None, None) == B.ATTN_OK


def test_status_strings():
    assert B.status_string(B.ATTN_OK) == "ok"
    assert "invalid" in B.status_string(B.ATTN_EINVAL)
    assert "unsupported" in B.status_string(B.ATTN_EUNSUPPORTED)


FAKE2 = ctypes.c_void_p(0x2000)


def shared_problem(**kw):
    p = B.attn_problem_t()
    B.lib().attn_problem_init(ctypes.byref(p), 1, 8, 1, 64, 64, 512, 512)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def bwd(p, k, v, dv, bias=None, flags=B.ATTN_SHARED_KV):
    return B.lib().attn_bwd(ctypes.byref(p), FAKE, k, v, FAKE, FAKE, FAKE, bias, FAKE, FAKE, dv, None, flags,
                            None)


def test_shared_kv_validation():
    p = shared_problem()
    # head dim 512 needs the shared-KV flag
    assert bwd(p, FAKE, FAKE, None, flags=0) == B.ATTN_EUNSUPPORTED
    # the flag needs one tensor: same pointer, same strides
    assert bwd(p, FAKE, FAKE2, None) == B.ATTN_EINVAL
    p2 = shared_problem()
    p2.v_str[2] = 1024
    assert bwd(p2, FAKE, FAKE, None) == B.ATTN_EINVAL
    # dk is the shared gradient: dv must be null
    assert bwd(p, FAKE, FAKE, FAKE) == B.ATTN_EINVAL
    # no bias, bf16 only, head dim 512 only
    assert bwd(p, FAKE, FAKE, None, bias=FAKE) == B.ATTN_EUNSUPPORTED
    assert bwd(shared_problem(in_dtype=B.ATTN_F32), FAKE, FAKE, None) == B.ATTN_EUNSUPPORTED
    assert bwd(problem(), FAKE, FAKE, None) == B.ATTN_EUNSUPPORTED
    # unaligned operand
    assert bwd(p, ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1008), None) == B.ATTN_EUNSUPPORTED
    # nothing to do: no device access
    assert bwd(shared_problem(B=0), FAKE, FAKE, None) == B.ATTN_OK


def test_shared_kv_forward_validation():
    L = B.lib()
    p = shared_problem()
    fwd = lambda p, k, v, bias=None: L.attn_fwd_lse(ctypes.byref(p), FAKE, k, v, bias, None, FAKE, FAKE,  # noqa: E731
                                                    None)
    assert fwd(p, FAKE, FAKE2) == B.ATTN_EUNSUPPORTED           # separate K and V at head dim 512
    assert fwd(p, FAKE, FAKE, bias=FAKE) == B.ATTN_EUNSUPPORTED
    assert fwd(shared_problem(in_dtype=B.ATTN_F32), FAKE, FAKE) == B.ATTN_EUNSUPPORTED
    assert fwd(shared_problem(Dv=256), FAKE, FAKE) == B.ATTN_EUNSUPPORTED
    assert fwd(shared_problem(Sq=0), FAKE, FAKE) == B.ATTN_OK


def sized_problem(B_, Hq, Hk, Sq, Sk, D, mask, **kw):
    p = B.attn_problem_t()
    B.lib().attn_problem_init(ctypes.byref(p), B_, Hq, Hk, Sq, Sk, D, D)
    p.mask = B.MASKS[mask]
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_workspace_size_query():
    """attn_bwd_workspace_size is host-only: 0 when no key block splits into
    more than two parts (the headline: two parts add onto zero), whole
    slots of 128 keys x (Dqk + Dv) floats per (batch entry, KV head) when
    one does (the small GQA workload splits eight ways), and 0 for paths
    without partial sums (fp32 inputs, a packed batch is not asked here)."""
    head = sized_problem(1, 32, 8, 4096, 4096, 128, "bottom_right")
    assert B.attn_bwd_workspace_size(head, 0) == 0
    # two parts added into existing values deterministically need slots
    assert B.attn_bwd_workspace_size(head, B.ATTN_DETERMINISTIC | B.ATTN_ACCUMULATE_DKDV) > 0
    small = sized_problem(2, 16, 4, 1024, 1024, 128, "top_left")
    n = B.attn_bwd_workspace_size(small, 0)
    slot = 128 * (128 + 128) * 4
    assert n > 0 and n % (2 * 4 * slot) == 0
    assert B.attn_bwd_workspace_size(small, B.ATTN_DETERMINISTIC) == n
    f32 = sized_problem(2, 16, 4, 1024, 1024, 128, "top_left", in_dtype=B.ATTN_F32)
    assert B.attn_bwd_workspace_size(f32, 0) == 0
    L = B.lib()
    assert L.attn_bwd_workspace_size(ctypes.byref(small), 0, None) == B.ATTN_EINVAL
    bad = sized_problem(2, 16, 3, 1024, 1024, 128, "top_left")   # Hq % Hk != 0
    x = ctypes.c_int64(7)
    assert L.attn_bwd_workspace_size(ctypes.byref(bad), 0, ctypes.byref(x)) == B.ATTN_EINVAL and x.value == 0
    assert L.attn_bwd_workspace_size(ctypes.byref(small), 64, ctypes.byref(x)) == B.ATTN_EINVAL


def test_workspace_size_other_paths():
    """The window + sink workload splits only its sink key block (parts
    summed through slots of that block alone); a packed batch and a bias
    problem keep atomic parts (0); the shared-KV head-dim-512 path sizes
    one dKV-shaped slot per query-head part beyond the first."""
    from attention_backward_attn_amd.inputs import WORKLOADS
    w = WORKLOADS["gqa8_swa1024_sink4_s8192"]
    p = sized_problem(w.B, w.Hq, w.Hk, w.Sq, w.Sk, w.Dqk, w.mask, window_left=w.window_left,
                      window_right=w.window_right, num_sink_tokens=w.num_sink)
    n = B.attn_bwd_workspace_size(p, 0)
    slot = 128 * (w.Dqk + w.Dv) * 4
    assert n > 0 and n % (w.B * w.Hk * slot) == 0
    # only the sink block's parts beyond the first (never more than 15 slots per head)
    assert n // (w.B * w.Hk * slot) <= 15
    # shared KV at head dim 512: (parts - 1) copies of the [Sk, Hk, 512] fp32 tensor
    kv = sized_problem(1, 64, 1, 4096, 4096, 512, "bottom_right", window_left=511)
    m = B.attn_bwd_workspace_size(kv, B.ATTN_SHARED_KV)
    one = 4096 * 512 * 4
    assert m > 0 and m % one == 0 and m // one in (1, 3, 7, 15)


def test_bwd_rejects_overlapping_dbias_strides():
    """dbias is written through the bias strides: rows or heads that overlap
    (a broadcast bias with stride 0, or a row stride below Sk) are rejected
    when dbias is asked for, and accepted for reading a bias alone."""
    L = B.lib()

    def call(bias_str, dbias):
        p = problem()
        p.bias_str[:] = bias_str
        # Sk = 0 and B = 0: no kernel would run even if validation passed
        return L.attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          FAKE if dbias else None, 0, None)

    for bad in ((0, 0), (64 * 64, 0), (0, 64), (64 * 63, 64), (64 * 64, 63)):
        assert call(bad, True) == B.ATTN_EINVAL, bad
    # a padded layout keeps rows and heads apart
    for good in ((64 * 64, 64), (65 * 72, 72)):
        p = problem(B=0)
        p.bias_str[:] = good
        assert L.attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                          None) == B.ATTN_OK, good
    # reading a broadcast bias without its gradient is fine
    p = problem(B=0)
    p.bias_str[:] = (0, 0)
    assert L.attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                      None) == B.ATTN_OK


def test_binding_checks_bias_shape():
    torch = pytest.importorskip("torch")
    q = torch.empty(1, 4, 64, 64, dtype=torch.bfloat16)
    k = torch.empty(1, 2, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.make_problem(q, k, k, bias=torch.empty(4, 64, 32))
    B.make_problem(q, k, k, bias=torch.empty(4, 64, 64))


def test_static_entry_point_rejects_oversized_problem():
    """attn_bwd_static refuses, before any HIP call, a problem whose partial
    sums need more than its static scratch (here 84 MiB: one KV head of
    12288 keys split eight ways); invalid arguments fail as in attn_bwd."""
    L = B.lib()
    p = B.attn_problem_t()
    L.attn_problem_init(ctypes.byref(p), 1, 8, 1, 12288, 12288, 128, 128)
    p.mask = 1
    n = ctypes.c_int64(0)
    assert L.attn_bwd_workspace_size(ctypes.byref(p), 0, ctypes.byref(n)) == B.ATTN_OK
    assert n.value > B.ATTN_STATIC_SCRATCH_BYTES
    args = [FAKE] * 7 + [FAKE, FAKE, FAKE, None, 0, None]
    assert L.attn_bwd_static(ctypes.byref(p), *args) == B.ATTN_ENOSCRATCH
    assert B.status_string(B.ATTN_ENOSCRATCH) != "unknown status"
    # validation comes first: a null dq is ATTN_EINVAL whatever the size
    bad = [FAKE] * 7 + [None, FAKE, FAKE, None, 0, None]
    assert L.attn_bwd_static(ctypes.byref(p), *bad) == B.ATTN_EINVAL


def test_empty_tensor_strides_read_as_dense():
    """Tensors with no elements (numpy gives them zero strides) are marshalled
    with dense strides, so an empty batch passes validation: attn_bwd with
    B = 0 returns ATTN_OK without touching the GPU."""
    torch = pytest.importorskip("torch")
    q = torch.from_numpy(np.zeros((0, 4, 70, 64), np.float32))
    k = torch.from_numpy(np.zeros((0, 2, 50, 64), np.float32))
    assert q.stride() == (0, 0, 0, 0)
    p = B.make_problem(q, k, k.clone(), o=q, do=q, dq=q, dk=k, dv=k, scale=0.125, mask="top_left")
    assert tuple(p.q_str) == (4 * 70 * 64, 70 * 64, 64) and tuple(p.k_str) == (2 * 50 * 64, 50 * 64, 64)
    assert B.lib().attn_bwd(ctypes.byref(p), None, None, None, None, None, None, None, None, None, None,
                            None, 0, None) == B.ATTN_OK
    t = torch.from_numpy(np.zeros((0, 4, 64), np.float32))   # packed [T, H, D]
    assert B._strides_packed(t) == (0, 64, 4 * 64)
