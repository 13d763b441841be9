"""fp64 CPU oracle: attention forward (O, LSE), backward (dQ, dK, dV, dbias,
dsinks), the preprocess row reduction and the log-sum-exp merge.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Notation follows the pages: B batch, Hq query heads, Hk key/value heads,
G = Hq / Hk query heads per KV head, Sq / Sk sequence lengths, Dqk / Dv head
dims.  Query head ``h`` reads KV head ``h // G`` ([GQA-BWD], K/V expanded with
``np.repeat`` along the head axis and dK/dV summed back with a
``reshape(B, Hk, G, ...)`` sum).  All arithmetic is fp64; inputs of any float
dtype are widened first.  Row ``i`` is a query position, column ``j`` a key
position.

How each function is pinned (tests/test_oracle_*.py):

==================  =========================================================
``allowed_mask``    brute-force loops written from [SINK] make_causal_mask /
                    make_causal_sink_mask / make_sliding_window_sink_mask and
                    the [SFMG] bottom-right ``threshold`` rule
``forward``         torch fp64 ``scaled_dot_product_attention`` (library) for
                    every mask, bias and GQA ratio; a sink logit through the
                    library as an extra zero-value key; closed forms Q = 0
                    and Sk = 1
``backward``        central finite differences of L = sum(O * dO) on every
                    input element ([DBIAS] Step 4 protocol, tightened for
                    fp64); torch fp64 autograd through the library SDPA;
                    invariants (zero dS row sums, sum_j dK = 0,
                    sum_j dV = sum_i dO, sinks shift invariance); GQA ==
                    expanded MHA ([GQA-BWD]); Sk = 1 special case
``preprocess``      the same FD pins (it is the D / dsinks part of backward)
``forward_varlen``  equal-length packed batch == the dense batch; each
``backward_varlen`` sequence == the dense oracle on that sequence alone
                    (a sequence's rows never see another's keys); empty
                    sequences contribute nothing
``lse_merge``       merged chunk forwards equal the unchunked forward;
                    identity with an empty partial; commutativity
``dq_rows`` /       equality with the corresponding rows / keys of
``dkdv_keys``       ``backward`` on small inputs
``backward_shared_  central finite differences of L = sum(O * dO) with the one
kv`` (+ ``_varlen``)  tensor perturbed in both roles; torch fp64 autograd
                    with one leaf tensor passed as keys and values; dK alone
                    (the dV term dropped) fails the finite-difference pin
==================  =========================================================

Readings of the pages that the code takes (each is listed with its reason in
the design notes): masked logits are -inf (not float32 min) so that a row
with no allowed key is empty (O = 0, LSE = -inf, zero gradients); sink
tokens are visible to every row, also to rows before them; a sliding window
of width W keeps keys [i - W + 1, i]; bottom-right alignment shifts the
diagonal by Sk_total - Sq_total; the sink logit is added to the scaled
logits of its query head and counted in LSE; dbias is the unscaled dS summed
over the batch; dsinks is summed over rows and batch.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

NEG_INF = -np.inf


@dataclass(frozen=True)
class MaskSpec:
    """Which (query, key) pairs may attend.

    kind:           'none' | 'top_left' | 'bottom_right'
    window_left:    -1 = unbounded; otherwise keys j >= i + delta - window_left
    window_right:   keys j <= i + delta + window_right (0 = causal)
    num_sink:       keys with global index < num_sink are always visible
    q_offset/k_offset: global index of local query row 0 / key 0 (chunking)
    sq_total/sk_total: global lengths used for bottom-right alignment
                    (None = the local lengths)
    """

    kind: str = "none"
    window_left: int = -1
    window_right: int = 0
    num_sink: int = 0
    q_offset: int = 0
    k_offset: int = 0
    sq_total: Optional[int] = None
    sk_total: Optional[int] = None


def allowed_mask(rows, cols, sq: int, sk: int, spec: MaskSpec) -> np.ndarray:
    """Boolean allowed(i, j) for local row indices ``rows`` and key indices
    ``cols`` (broadcast against each other).

    [SINK] make_causal_mask: top-left causal keeps j <= i.
    [SINK] make_causal_sink_mask / make_sliding_window_sink_mask: keys
    j < num_sink are always attended; a window W keeps i - W + 1 <= j <= i,
    i.e. window_left = W - 1, window_right = 0.
    [SFMG] "Example": under bottom-right alignment query s1 may use keys
    below delta_s + s1 + 1 with delta_s = S2 - S1, i.e. j <= i + (Sk - Sq).
    """
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    if spec.kind == "none":
        return np.ones(np.broadcast(rows, cols).shape, dtype=bool)
    sq_total = sq if spec.sq_total is None else spec.sq_total
    sk_total = sk if spec.sk_total is None else spec.sk_total
    if spec.kind == "top_left":
        delta = 0
    elif spec.kind == "bottom_right":
        delta = sk_total - sq_total
    else:
        raise ValueError(f"unknown mask kind {spec.kind!r}")
    i = rows + spec.q_offset
    j = cols + spec.k_offset
    ok = j <= i + delta + spec.window_right
    if spec.window_left >= 0:
        ok = ok & (j >= i + delta - spec.window_left)
    if spec.num_sink > 0:
        ok = ok | (j < spec.num_sink)
    return ok


def allowed_pair_count(sq: int, sk: int, spec: MaskSpec, row_block: int = 1024) -> int:
    """Exact number of allowed (i, j) pairs for one head, by brute force over
    the dense predicate (the attention-density measurement of [SINK])."""
    total = 0
    cols = np.arange(sk)[None, :]
    for r0 in range(0, sq, row_block):
        rows = np.arange(r0, min(sq, r0 + row_block))[:, None]
        total += int(allowed_mask(rows, cols, sq, sk, spec).sum())
    return total


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _block_logits(q_rows, k_all, h, rows, scale, spec, sq, sk, bias):
    """Scaled logits of ``q_rows`` against the key columns that are allowed
    for at least one of ``rows``: S = scale * Q K^T (+ bias), -inf where
    masked ([GQA-BWD] cpu_fwd_with_intermediates, [DBIAS]
    cpu_attention_fwd_bias, [SINK] cpu_attention_fwd_masked).  Restricting to
    those columns is exact: every other column has P = 0 on these rows.
    Returns (cols, s, allowed)."""
    m = allowed_mask(rows[:, None], np.arange(sk)[None, :], sq, sk, spec)
    cols = np.nonzero(m.any(axis=0))[0]
    m = m[:, cols]
    s = scale * (q_rows @ k_all[cols].T)
    if bias is not None:
        s = s + bias[h][np.ix_(rows, cols)]
    s = np.where(m, s, NEG_INF)
    return cols, s, m


def forward(q, k, v, scale: float, spec: MaskSpec = MaskSpec(), bias=None, sinks=None,
            row_block: int = 512):
    """Attention forward returning (O, LSE) in fp64.

    S = scale * Q K^T + bias (masked to -inf); the optional per-head sink
    logit joins the softmax denominator but has no value row;
    LSE_i = m_i + log(sum_j e^{S_ij - m_i} + e^{sink - m_i}) with
    m_i = max(max_j S_ij, sink); P = e^{S - LSE}; O = P V.  A row with no
    allowed key and no sink has O = 0 and LSE = -inf.

    [GQA-BWD] cpu_fwd_with_intermediates (stable softmax with max subtraction,
    lse = log(sum) + max); [DBIAS] cpu_attention_fwd_bias (bias [H, Sq, Sk]
    broadcast over batch); [SINK] cpu_attention_fwd_masked; [SFMG] Phase 3
    (the sink logit inside the softmax normaliser, SimpleSoftmax(sinks, lse)).
    """
    q, k, v, bias, sinks = _f64(q), _f64(k), _f64(v), _f64(bias), _f64(sinks)
    B, Hq, Sq, _ = q.shape
    Hk, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hk
    o = np.zeros((B, Hq, Sq, Dv))
    lse = np.full((B, Hq, Sq), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, Sq, row_block):
                rows = np.arange(r0, min(Sq, r0 + row_block))
                cols, s, _ = _block_logits(q[b, h, rows], k[b, g], h, rows, scale, spec, Sq, Sk, bias)
                mx = s.max(axis=1) if cols.size else np.full(rows.size, NEG_INF)
                if sinks is not None:
                    mx = np.maximum(mx, sinks[h])
                live = np.isfinite(mx)
                mxs = np.where(live, mx, 0.0)
                e = np.where(live[:, None], np.exp(s - mxs[:, None]), 0.0)
                den = e.sum(axis=1)
                if sinks is not None:
                    den = den + np.exp(sinks[h] - mxs)
                safe = np.where(live, den, 1.0)
                p = e / safe[:, None]
                o[b, h, rows] = p @ v[b, g, cols] if cols.size else 0.0
                lse[b, h, rows] = np.where(live, mxs + np.log(safe), NEG_INF)
    return o, lse


def preprocess(o, do, lse, sinks=None):
    """D = rowsum(dO * O) per (b, h, i) ([GQA-BWD] cpu_bwd_gqa:
    ``D = (dO * out).sum(-1)``; [SFMG] Phase 2: SoftmaxGrad(dO, O)) and
    dsinks[h] = -sum_{b,i} e^{sink_h - LSE_bhi} * D_bhi ([SFMG] Phase 3 dSinks:
    -P * dP * SimpleSoftmax(sinks, lse) reduced over the keys of a row gives
    -p_sink,i * D_i; reduced again over rows and batch to the shape of sinks).
    Rows with LSE = -inf contribute nothing."""
    o, do, lse, sinks = _f64(o), _f64(do), _f64(lse), _f64(sinks)
    delta = (do * o).sum(axis=-1)
    dsinks = None
    if sinks is not None:
        live = np.isfinite(lse)
        psink = np.where(live, np.exp(sinks[None, :, None] - np.where(live, lse, 0.0)), 0.0)
        dsinks = -(psink * delta).sum(axis=(0, 2))
    return delta, dsinks


def backward(q, k, v, o, do, lse, scale: float, spec: MaskSpec = MaskSpec(), bias=None,
             sinks=None, row_block: int = 512):
    """Attention backward given the saved O and LSE.

    P = e^{S - LSE} on allowed pairs (0 elsewhere and on rows with
    LSE = -inf); dP = dO V^T; D = rowsum(dO * O); dS = P * (dP - D);
    dQ = scale * dS K; dK = scale * dS^T Q and dV = P^T dO, each summed over
    the G query heads of a KV head; dbias = sum_b dS (unscaled);
    dsinks as in ``preprocess``.

    [GQA-BWD] module docstring and cpu_bwd_gqa; [DBIAS] cpu_attention_bwd_dbias
    (scale folded into dS there and divided back out for dbias, so dbias is
    the unscaled dS summed over batch); [SFMG] Phase 2 and Phase 3.
    Returns a dict with dq, dk, dv, dbias (or None), dsinks (or None), delta.
    """
    q, k, v, o, do, lse = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do), _f64(lse)
    bias, sinks = _f64(bias), _f64(sinks)
    B, Hq, Sq, Dqk = q.shape
    Hk, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hk
    delta, dsinks = preprocess(o, do, lse, sinks)
    dq = np.zeros_like(q)
    dk = np.zeros((B, Hk, Sk, Dqk))
    dv = np.zeros((B, Hk, Sk, Dv))
    dbias = np.zeros((Hq, Sq, Sk)) if bias is not None else None
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, Sq, row_block):
                rows = np.arange(r0, min(Sq, r0 + row_block))
                cols, s, m = _block_logits(q[b, h, rows], k[b, g], h, rows, scale, spec, Sq, Sk, bias)
                if cols.size == 0:
                    continue
                l_i = lse[b, h, rows]
                live = np.isfinite(l_i)
                p = np.where(m & live[:, None], np.exp(s - np.where(live, l_i, 0.0)[:, None]), 0.0)
                dp = do[b, h, rows] @ v[b, g, cols].T
                ds = p * (dp - delta[b, h, rows][:, None])
                dq[b, h, rows] = scale * (ds @ k[b, g, cols])
                dk[b, g, cols] += scale * (ds.T @ q[b, h, rows])
                dv[b, g, cols] += p.T @ do[b, h, rows]
                if dbias is not None:
                    dbias[np.ix_([h], rows, cols)] += ds[None]
    return {"dq": dq, "dk": dk, "dv": dv, "dbias": dbias, "dsinks": dsinks, "delta": delta}


def dq_rows(q, k, v, o, do, lse, scale, spec, b, h, rows, bias=None):
    """dQ[b, h, rows] alone (same definition as ``backward``), for sampled
    checks at sizes where the full backward is too slow."""
    q, k, v, o, do, lse, bias = (_f64(x) for x in (q, k, v, o, do, lse, bias))
    Sq, Sk = q.shape[2], k.shape[2]
    G = q.shape[1] // k.shape[1]
    g = h // G
    rows = np.asarray(rows)
    cols, s, m = _block_logits(q[b, h, rows], k[b, g], h, rows, scale, spec, Sq, Sk, bias)
    out = np.zeros((rows.size, q.shape[3]))
    if cols.size == 0:
        return out
    l_i = lse[b, h, rows]
    live = np.isfinite(l_i)
    p = np.where(m & live[:, None], np.exp(s - np.where(live, l_i, 0.0)[:, None]), 0.0)
    d_i = (do[b, h, rows] * o[b, h, rows]).sum(axis=-1)
    ds = p * (do[b, h, rows] @ v[b, g, cols].T - d_i[:, None])
    return scale * (ds @ k[b, g, cols])


def ds_rows(q, k, v, o, do, lse, scale, spec, b, h, rows, bias=None):
    """dS[b, h, rows, :] over every key (0 where masked), the unscaled
    gradient of the logits; dbias rows are its sum over the batch."""
    q, k, v, o, do, lse, bias = (_f64(x) for x in (q, k, v, o, do, lse, bias))
    Sq, Sk = q.shape[2], k.shape[2]
    G = q.shape[1] // k.shape[1]
    g = h // G
    rows = np.asarray(rows)
    out = np.zeros((rows.size, Sk))
    cols, s, m = _block_logits(q[b, h, rows], k[b, g], h, rows, scale, spec, Sq, Sk, bias)
    if cols.size == 0:
        return out
    l_i = lse[b, h, rows]
    live = np.isfinite(l_i)
    p = np.where(m & live[:, None], np.exp(s - np.where(live, l_i, 0.0)[:, None]), 0.0)
    d_i = (do[b, h, rows] * o[b, h, rows]).sum(axis=-1)
    out[:, cols] = p * (do[b, h, rows] @ v[b, g, cols].T - d_i[:, None])
    return out


def dkdv_keys(q, k, v, o, do, lse, scale, spec, b, g, keys, bias=None):
    """(dK, dV)[b, g, keys] alone: every query row of every query head in
    KV head g's group against the chosen keys (same definition as
    ``backward``)."""
    q, k, v, o, do, lse, bias = (_f64(x) for x in (q, k, v, o, do, lse, bias))
    Hq, Sq, Dqk = q.shape[1], q.shape[2], q.shape[3]
    Sk, Dv = k.shape[2], v.shape[3]
    G = Hq // k.shape[1]
    keys = np.asarray(keys)
    dk = np.zeros((keys.size, Dqk))
    dv = np.zeros((keys.size, Dv))
    rows = np.arange(Sq)
    m = allowed_mask(rows[:, None], keys[None, :], Sq, Sk, spec)
    for h in range(g * G, (g + 1) * G):
        s = scale * (q[b, h] @ k[b, g, keys].T)
        if bias is not None:
            s = s + bias[h][:, keys]
        l_i = lse[b, h]
        live = np.isfinite(l_i)
        p = np.where(m & live[:, None], np.exp(np.where(m, s, 0.0) - np.where(live, l_i, 0.0)[:, None]), 0.0)
        d_i = (do[b, h] * o[b, h]).sum(axis=-1)
        ds = p * (do[b, h] @ v[b, g, keys].T - d_i[:, None])
        dk += scale * (ds.T @ q[b, h])
        dv += p.T @ do[b, h]
    return dk, dv


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two partial attention results over disjoint key sets:
    lse = logaddexp(lse_a, lse_b); o = o_a e^{lse_a - lse} + o_b e^{lse_b - lse}
    ([RING] _ring_fwd).  When both parts are empty (lse = -inf) the result is
    o = 0, lse = -inf (the gist's expression would give NaN there)."""
    o_a, lse_a, o_b, lse_b = _f64(o_a), _f64(lse_a), _f64(o_b), _f64(lse_b)
    lse = np.logaddexp(lse_a, lse_b)
    live = np.isfinite(lse)
    safe = np.where(live, lse, 0.0)
    wa = np.where(live & np.isfinite(lse_a), np.exp(np.where(np.isfinite(lse_a), lse_a, 0.0) - safe), 0.0)
    wb = np.where(live & np.isfinite(lse_b), np.exp(np.where(np.isfinite(lse_b), lse_b, 0.0) - safe), 0.0)
    o = o_a * wa[..., None] + o_b * wb[..., None]
    return o, lse


def _unpack(x, c0, c1):
    """Rows [c0, c1) of a packed [T, H, D] tensor as a [1, H, c1 - c0, D] batch."""
    return x[c0:c1].transpose(1, 0, 2)[None]


def forward_varlen(q, k, v, cu_q, cu_k, max_q: int, scale: float, spec: MaskSpec = MaskSpec(),
                   sinks=None):
    """Forward of a variable-length packed batch ([SFMG] "Prototype": TND
    layout with cumulative sequence lengths).  q: [Tq, Hq, D], k / v:
    [Tk, Hk, D]; sequence b owns rows cu_q[b]..cu_q[b+1] and keys
    cu_k[b]..cu_k[b+1], and attends to its own keys only, with masks aligned
    on its own lengths.  Returns packed O [Tq, Hq, Dv] and LSE [B, Hq, max_q]
    (rows past a sequence's length stay -inf)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B = len(cu_q) - 1
    o = np.zeros((q.shape[0], q.shape[1], v.shape[2]))
    lse = np.full((B, q.shape[1], max_q), NEG_INF)
    for b in range(B):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0:
            continue
        ob, lb = forward(_unpack(q, q0, q1), _unpack(k, k0, k1), _unpack(v, k0, k1), scale, spec, None, sinks)
        o[q0:q1] = ob[0].transpose(1, 0, 2)
        lse[b, :, :q1 - q0] = lb[0]
    return o, lse


def backward_varlen(q, k, v, o, do, lse, cu_q, cu_k, scale: float, spec: MaskSpec = MaskSpec(),
                    sinks=None):
    """Backward of a variable-length packed batch: each sequence is the dense
    problem on its own rows and keys (see ``forward_varlen``).  Packed dq
    [Tq, Hq, Dqk], dk / dv [Tk, Hk, D]; delta [B, Hq, max_q] (0 past a
    sequence's length); dsinks summed over every sequence's rows."""
    q, k, v, o, do, lse = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do), _f64(lse)
    B = len(cu_q) - 1
    dq, dk, dv = np.zeros_like(q), np.zeros(k.shape), np.zeros(v.shape)
    delta = np.zeros(lse.shape)
    dsinks = None if sinks is None else np.zeros(q.shape[1])
    for b in range(B):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0 and k1 == k0:
            continue
        n = q1 - q0
        g = backward(_unpack(q, q0, q1), _unpack(k, k0, k1), _unpack(v, k0, k1), _unpack(o, q0, q1),
                     _unpack(do, q0, q1), lse[b:b + 1, :, :n], scale, spec, None, sinks)
        dq[q0:q1] = g["dq"][0].transpose(1, 0, 2)
        dk[k0:k1] = g["dk"][0].transpose(1, 0, 2)
        dv[k0:k1] = g["dv"][0].transpose(1, 0, 2)
        delta[b, :, :n] = g["delta"][0]
        if dsinks is not None and n > 0:
            dsinks += g["dsinks"]
    return {"dq": dq, "dk": dk, "dv": dv, "dsinks": dsinks, "delta": delta}


def backward_shared_kv(q, kv, o, do, lse, scale: float, spec: MaskSpec = MaskSpec(), sinks=None,
                       row_block: int = 512):
    """Backward when one tensor ``kv`` [B, Hk, Sk, D] serves as keys and
    values ([SFMG] "Formula", sliding-window case: the selected KV is the
    original KV, used in Q KV^T, dO KV^T and dS KV).  Its gradient collects
    both uses, dKV = scale * dS^T Q + P^T dO ([SFMG] Phase 3): by the chain
    rule, the dK plus the dV of ``backward`` with k = v = kv.  Returns a dict
    with dq, dkv, dsinks (or None) and delta."""
    g = backward(q, kv, kv, o, do, lse, scale, spec, None, sinks, row_block)
    return {"dq": g["dq"], "dkv": g["dk"] + g["dv"], "dsinks": g["dsinks"], "delta": g["delta"]}


def backward_shared_kv_varlen(q, kv, o, do, lse, cu_q, cu_k, scale: float, spec: MaskSpec = MaskSpec(),
                              sinks=None):
    """``backward_shared_kv`` of a variable-length packed batch (TND, see
    ``forward_varlen``): packed dq [Tq, Hq, D] and dkv [Tk, Hk, D]."""
    g = backward_varlen(q, kv, kv, o, do, lse, cu_q, cu_k, scale, spec, sinks)
    return {"dq": g["dq"], "dkv": g["dk"] + g["dv"], "dsinks": g["dsinks"], "delta": g["delta"]}
