"""ctypes binding of libattnbwd.so: the C ABI's entry points under the same
names, taking torch tensors for device memory and a torch stream.

This layer only marshals arguments (tensor pointers, strides, stream
handles) -- every step of the computation runs in the HIP kernels behind
the C ABI.  If the compiled library is missing the first call raises; there
is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattnbwd.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP, ATTN_ENOSCRATCH = 0, -1, -2, -3, -4
ATTN_STATIC_SCRATCH_BYTES = 64 * 1024 * 1024
ATTN_F32, ATTN_BF16 = 0, 1
MASKS = {"none": 0, "top_left": 1, "bottom_right": 2}
ATTN_DETERMINISTIC, ATTN_ACCUMULATE_DQ, ATTN_ACCUMULATE_DKDV, ATTN_SHARED_KV = 1, 2, 4, 8

EXPORTED = ("attn_problem_init", "attn_fwd_lse", "attn_bwd_preprocess", "attn_bwd", "attn_bwd_static",
            "attn_bwd_workspace_size", "attn_lse_merge", "attn_status_string")


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class attn_problem_t(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hk", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32),
        ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32), ("mask", ctypes.c_int32),
        ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
        ("num_sink_tokens", ctypes.c_int32),
        ("q_offset", ctypes.c_int64), ("k_offset", ctypes.c_int64),
        ("sq_total", ctypes.c_int64), ("sk_total", ctypes.c_int64),
        ("q_str", ctypes.c_int64 * 3), ("k_str", ctypes.c_int64 * 3), ("v_str", ctypes.c_int64 * 3),
        ("o_str", ctypes.c_int64 * 3), ("do_str", ctypes.c_int64 * 3),
        ("dq_str", ctypes.c_int64 * 3), ("dk_str", ctypes.c_int64 * 3), ("dv_str", ctypes.c_int64 * 3),
        ("bias_str", ctypes.c_int64 * 2),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
    ]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load the compiled library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m attention_backward_attn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, fp, i32, i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64  # noqa: F841
        P = ctypes.POINTER(attn_problem_t)
        L.attn_problem_init.argtypes = [P] + [i32] * 7
        L.attn_problem_init.restype = None
        L.attn_fwd_lse.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_fwd_lse.restype = i32
        L.attn_bwd_preprocess.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_bwd_preprocess.restype = i32
        L.attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp]
        L.attn_bwd.restype = i32
        L.attn_bwd_static.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp]
        L.attn_bwd_static.restype = i32
        L.attn_bwd_workspace_size.argtypes = [P, ctypes.c_uint32, ctypes.POINTER(i64)]
        L.attn_bwd_workspace_size.restype = i32
        L.attn_lse_merge.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.attn_lse_merge.restype = i32
        L.attn_status_string.argtypes = [i32]
        L.attn_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def status_string(s: int) -> str:
    return lib().attn_status_string(s).decode()


def _check(fn: str, s: int):
    if s != ATTN_OK:
        raise AttnError(fn, s, status_string(s))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dense_strides(shape):
    st = [1] * len(shape)
    for i in range(len(shape) - 2, -1, -1):
        st[i] = st[i + 1] * max(int(shape[i + 1]), 1)
    return st


def _strides3(t):
    if t is None:
        return (0, 0, 0)
    if t.numel() == 0:   # no element is addressed: any strides (numpy gives zeros) read as dense
        return tuple(_dense_strides(t.shape)[:3])
    if t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    return tuple(t.stride()[:3])


def _strides_packed(t):
    """{b, h, s} strides of a packed [T, H, D] tensor (the b stride is unused)."""
    if t is None:
        return (0, 0, 0)
    if t.numel() == 0:
        st = _dense_strides(t.shape)
        return (0, st[1], st[0])
    if t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    return (0, t.stride(1), t.stride(0))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def make_problem(q, k, v, *, o=None, do=None, dq=None, dk=None, dv=None, bias=None,
                 scale: Optional[float] = None, mask: str = "none", window_left: int = -1,
                 window_right: int = 0, num_sink_tokens: int = 0, q_offset: int = 0,
                 k_offset: int = 0, sq_total: int = 0, sk_total: int = 0,
                 cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q: int = 0,
                 max_seqlen_k: int = 0) -> attn_problem_t:
    """Problem descriptor from tensors in [B, H, S, D] layout, or -- with
    cu_seqlens_q / cu_seqlens_k (int32 device tensors of B + 1 prefix sums)
    -- from packed [T, H, D] tensors of a variable-length batch (TND)."""
    packed = cu_seqlens_q is not None
    if packed:
        if cu_seqlens_k is None or q.dim() != 3:
            raise ValueError("a packed batch needs cu_seqlens_q, cu_seqlens_k and [T, H, D] tensors")
        B = cu_seqlens_q.numel() - 1
        Hq, Dqk = q.shape[1], q.shape[2]
        Hk, Dv = k.shape[1], v.shape[2]
        Sq, Sk = max_seqlen_q, max_seqlen_k
    else:
        B, Hq, Sq, Dqk = q.shape
        Hk, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    p = attn_problem_t()
    lib().attn_problem_init(ctypes.byref(p), B, Hq, Hk, Sq, Sk, Dqk, Dv)
    if packed:
        p.cu_seqlens_q, p.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
        p.total_q, p.total_k = q.shape[0], k.shape[0]
    if scale is not None:
        p.scale = float(scale)
    p.in_dtype = _dtype_code(q)
    p.o_dtype = _dtype_code(o) if o is not None else ATTN_F32
    p.mask = MASKS[mask]
    p.window_left, p.window_right, p.num_sink_tokens = window_left, window_right, num_sink_tokens
    p.q_offset, p.k_offset, p.sq_total, p.sk_total = q_offset, k_offset, sq_total, sk_total
    st = _strides_packed if packed else _strides3
    p.q_str[:] = st(q)
    p.k_str[:] = st(k)
    p.v_str[:] = st(v)
    if o is not None:
        p.o_str[:] = st(o)
    if do is not None:
        p.do_str[:] = st(do)
    if dq is not None:
        p.dq_str[:] = st(dq)
    if dk is not None:
        p.dk_str[:] = st(dk)
    if dv is not None:
        p.dv_str[:] = st(dv)
    if bias is not None:
        if tuple(bias.shape) != (Hq, Sq, Sk):
            raise ValueError(f"bias must be [Hq, Sq, Sk] = {(Hq, Sq, Sk)}, got {tuple(bias.shape)}")
        if bias.stride(-1) != 1:
            raise ValueError("bias: the key dimension must be contiguous")
        p.bias_str[:] = (bias.stride(0), bias.stride(1))
    return p


def attn_fwd_lse(p: attn_problem_t, q, k, v, bias, sinks, o, lse, stream=None):
    _check("attn_fwd_lse", lib().attn_fwd_lse(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                              _ptr(sinks), _ptr(o), _ptr(lse), _stream(stream)))


def attn_bwd_preprocess(p: attn_problem_t, o, do, lse, sinks, delta, dsinks, dq_zero=None, dk_zero=None,
                        dv_zero=None, stream=None):
    _check("attn_bwd_preprocess",
           lib().attn_bwd_preprocess(ctypes.byref(p), _ptr(o), _ptr(do), _ptr(lse), _ptr(sinks),
                                     _ptr(delta), _ptr(dsinks), _ptr(dq_zero), _ptr(dk_zero), _ptr(dv_zero),
                                     _stream(stream)))


def attn_bwd(p: attn_problem_t, q, k, v, do, lse, delta, bias, dq, dk, dv, dbias, flags: int = 0,
             stream=None):
    _check("attn_bwd", lib().attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
                                      _ptr(delta), _ptr(bias), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias),
                                      flags, _stream(stream)))


def attn_bwd_static(p: attn_problem_t, q, k, v, do, lse, delta, bias, dq, dk, dv, dbias, flags: int = 0,
                    stream=None):
    """attn_bwd with the library's static device scratch in place of
    p.workspace (allocates nothing)."""
    _check("attn_bwd_static",
           lib().attn_bwd_static(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta),
                                 _ptr(bias), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), flags, _stream(stream)))


def attn_bwd_workspace_size(p: attn_problem_t, flags: int = 0) -> int:
    """Bytes of caller workspace with which attn_bwd keeps split key blocks'
    partial sums (0: none used)."""
    n = ctypes.c_int64(0)
    _check("attn_bwd_workspace_size", lib().attn_bwd_workspace_size(ctypes.byref(p), flags, ctypes.byref(n)))
    return int(n.value)


def set_workspace(p: attn_problem_t, flags: int = 0, device=None, bias=None):
    """Attach a workspace of attn_bwd_workspace_size bytes to p (a torch
    uint8 tensor, returned so that the caller keeps it alive; None when the
    call needs none -- a problem with a bias uses none)."""
    n = 0 if bias is not None else attn_bwd_workspace_size(p, flags)
    if n == 0:
        p.workspace, p.workspace_bytes = None, 0
        return None
    import torch
    ws = torch.empty(n, dtype=torch.uint8, device=device or "cuda")
    p.workspace, p.workspace_bytes = ws.data_ptr(), n
    return ws


def _torch_stream(stream, device):
    """The torch stream object of a stream argument (None: the current one;
    a raw handle is wrapped)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def attn_lse_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    B, H, Sq, Dv = o_acc.shape
    for t in (o_acc, lse_acc, o_part, lse_part):
        if not t.is_contiguous():
            raise ValueError("attn_lse_merge needs contiguous buffers")
    _check("attn_lse_merge", lib().attn_lse_merge(B, H, Sq, Dv, _ptr(o_acc), _ptr(lse_acc), _ptr(o_part),
                                                  _ptr(lse_part), _stream(stream)))


# ---------------------------------------------------------------------------
# Convenience wrappers that allocate outputs with torch (device memory only).
# ---------------------------------------------------------------------------
def forward(q, k, v, *, bias=None, sinks=None, o_dtype=None, stream=None, **mask_kw):
    """(O, LSE) of attention; O in ``o_dtype`` (default fp32).  With
    cu_seqlens_q / cu_seqlens_k (packed [T, H, D] tensors) O is packed too
    and LSE is [B, Hq, max_seqlen_q]."""
    import torch
    if mask_kw.get("cu_seqlens_q") is not None:
        B, Hq, Sq = mask_kw["cu_seqlens_q"].numel() - 1, q.shape[1], mask_kw["max_seqlen_q"]
        o = torch.empty(q.shape[0], Hq, v.shape[2], device=q.device, dtype=o_dtype or torch.float32)
    else:
        B, Hq, Sq, _ = q.shape
        o = torch.empty(B, Hq, Sq, v.shape[3], device=q.device, dtype=o_dtype or torch.float32)
    lse = torch.empty(B, Hq, Sq, device=q.device, dtype=torch.float32)
    p = make_problem(q, k, v, o=o, bias=bias, **mask_kw)
    attn_fwd_lse(p, q, k, v, bias, sinks, o, lse, stream)
    return o, lse


def backward(q, k, v, o, do, lse, *, bias=None, sinks=None, want_dbias=False, flags=0, stream=None,
             dq=None, workspace: bool = True, **mask_kw):
    """Full backward: preprocess then the main pass.  Returns a dict with
    dq, dk, dv (fp32), dbias and dsinks (or None) and delta.  With
    ATTN_SHARED_KV in flags (k is v) dk is the gradient of the shared tensor
    and dv is None.  ``workspace`` False runs attn_bwd without a caller
    workspace (the parts of split key blocks then add atomically)."""
    import torch
    dev = q.device
    if mask_kw.get("cu_seqlens_q") is not None:
        B, Hq, Sq = mask_kw["cu_seqlens_q"].numel() - 1, q.shape[1], mask_kw["max_seqlen_q"]
    else:
        B, Hq, Sq, _ = q.shape
    dq = torch.empty(q.shape, device=dev, dtype=torch.float32) if dq is None else dq
    dk = torch.empty(k.shape, device=dev, dtype=torch.float32)
    # one tensor as keys and values: dk is the gradient of that tensor
    dv = None if flags & ATTN_SHARED_KV else torch.empty(v.shape, device=dev, dtype=torch.float32)
    delta = torch.empty(B, Hq, Sq, device=dev, dtype=torch.float32)
    dsinks = torch.empty(Hq, device=dev, dtype=torch.float32) if sinks is not None else None
    dbias = None
    if want_dbias and bias is not None:
        # dbias is written through the bias strides: give a strided or
        # broadcast bias a dense copy, so that dbias has the same layout
        if not bias.is_contiguous():
            bias = bias.contiguous()
        dbias = torch.empty(bias.shape, device=dev, dtype=torch.float32)
    p = make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, bias=bias, **mask_kw)
    # workspace for split key blocks' partial sums, marked as in use on the
    # call's stream: torch's caching allocator then hands the block to no
    # other allocation before that stream has finished the call
    ws = set_workspace(p, flags, dev, bias) if workspace else None
    if ws is not None:
        ws.record_stream(_torch_stream(stream, dev))
    attn_bwd_preprocess(p, o, do, lse, sinks, delta, dsinks, None, None, None, stream)
    attn_bwd(p, q, k, v, do, lse, delta, bias, dq, dk, dv, dbias, flags, stream)
    del ws
    return {"dq": dq, "dk": dk, "dv": dv, "dbias": dbias, "dsinks": dsinks, "delta": delta}
