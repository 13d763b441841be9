"""Host-side mask arithmetic: exact allowed-pair counts for the FLOP figure.

The mask is the one the kernels apply (CK FMHA example 22 "Sink Token
Attention FMHA" causal / sliding-window / sink-token masks; bottom-right
alignment from the CANN sparse_flash_mla_grad "Example"): in global indices
i' = q_offset + i, j' = k_offset + j and delta = 0 (top-left) or
sk_total - sq_total (bottom-right), a pair is allowed when

    i' + delta - window_left <= j' <= i' + delta + window_right   (window_left < 0: no lower bound)
    or j' < num_sink.

Counts are computed per row in closed form (interval lengths), not by
enumerating pairs.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

MASK_KINDS = {"none": 0, "top_left": 1, "bottom_right": 2}


def row_counts(sq: int, sk: int, kind: str, window_left: int = -1, window_right: int = 0,
               num_sink: int = 0, q_offset: int = 0, k_offset: int = 0,
               sq_total: Optional[int] = None, sk_total: Optional[int] = None) -> np.ndarray:
    """Number of allowed keys for each local query row (int64 array [sq])."""
    if kind == "none":
        return np.full(sq, sk, dtype=np.int64)
    sq_t = sq if sq_total is None else sq_total
    sk_t = sk if sk_total is None else sk_total
    delta = 0 if kind == "top_left" else sk_t - sq_t
    i = np.arange(sq, dtype=np.int64) + q_offset
    k_lo, k_hi = k_offset, k_offset + sk - 1            # local key range, global indices
    hi = np.minimum(i + delta + window_right, k_hi)
    lo = np.full(sq, k_lo, dtype=np.int64) if window_left < 0 else np.maximum(i + delta - window_left, k_lo)
    band = np.maximum(hi - lo + 1, 0)
    # sink keys inside this chunk: [k_lo, min(num_sink, k_hi + 1))
    s_hi = min(num_sink, k_hi + 1) - 1
    n_sink_local = max(s_hi - k_lo + 1, 0)
    if n_sink_local == 0:
        return band
    # sink keys already inside the band: |[lo, hi] intersect [k_lo, s_hi]|
    overlap = np.maximum(np.minimum(hi, s_hi) - np.maximum(lo, k_lo) + 1, 0)
    overlap = np.where(band > 0, overlap, 0)
    return band + n_sink_local - overlap


def allowed_pairs(sq: int, sk: int, kind: str, window_left: int = -1, window_right: int = 0,
                  num_sink: int = 0, q_offset: int = 0, k_offset: int = 0,
                  sq_total: Optional[int] = None, sk_total: Optional[int] = None) -> int:
    """Exact number of allowed (i, j) pairs of one head."""
    return int(row_counts(sq, sk, kind, window_left, window_right, num_sink, q_offset, k_offset,
                          sq_total, sk_total).sum())


def backward_flops(w, pairs_per_head: Optional[int] = None) -> float:
    """Counted backward FLOPs: 2 * (3 * Dqk + 2 * Dv) per allowed pair per query
    head -- the five contractions S = Q K^T, dP = dO V^T, dV = P^T dO,
    dK = dS^T Q and dQ = dS K, each 2 * D multiply-adds per pair.
    (= 10 * D when Dqk = Dv = D.)"""
    if pairs_per_head is None:
        pairs_per_head = allowed_pairs(w.Sq, w.Sk, w.mask, w.window_left, w.window_right, w.num_sink)
    return float(2 * (3 * w.Dqk + 2 * w.Dv)) * pairs_per_head * w.B * w.Hq


def backward_bytes(w) -> int:
    """Algorithmic HBM bytes of one attn_bwd call (the main pass, without the
    preprocess): every input read once and every output written once --
    Q, dO (B Hq Sq D) and K, V (B Hk Sk D) in the input dtype, LSE and delta
    (4 bytes per query row), the fp32 bias [Hq, Sq, Sk] when there is one;
    dQ, dK, dV in fp32 and dbias [Hq, Sq, Sk] in fp32 when there is a bias."""
    e = 2 if w.dtype == "bf16" else 4
    rows = w.B * w.Hq * w.Sq
    reads = e * (rows * (w.Dqk + w.Dv) + w.B * w.Hk * w.Sk * (w.Dqk + w.Dv)) + 8 * rows
    writes = 4 * (rows * w.Dqk + w.B * w.Hk * w.Sk * (w.Dqk + w.Dv))
    if w.bias:
        reads += 4 * w.Hq * w.Sq * w.Sk
        writes += 4 * w.Hq * w.Sq * w.Sk
    return int(reads + writes)
