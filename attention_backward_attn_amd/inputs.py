"""Seeded synthetic inputs for the five attention-backward workloads.

This module holds workload descriptions and random draws only -- none of the
attention arithmetic.  It is shared by the parity tests (which hand the same
arrays to the CPU oracle and to the HIP library) and by ``bench.py``.

Recipe: ``numpy.random.default_rng(seed)`` draws Q, K, V, dO and then the
per-head sink logits, each ``standard_normal`` in float64, narrowed to
float32 and, for bf16 workloads, rounded to bf16 with round-to-nearest-even
(the values stay in float32 arrays; every one is exactly representable in
bf16).  Layout is [B, H, S, D] contiguous.  The ALiBi bias follows
``make_alibi_bias`` of CK FMHA example 28 ("Backward Bias Gradient (dbias)
FMHA"): slope_h = 2^(-8 (h + 1) / H), bias[h, i, j] = -slope_h * |i - j|,
computed in float64 and stored float32, shared over the batch.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One attention-backward problem: shapes, input dtype, mask and extras."""

    name: str
    B: int
    Hq: int
    Hk: int
    Sq: int
    Sk: int
    Dqk: int
    Dv: int
    dtype: str                      # 'f32' | 'bf16'  (Q, K, V, dO)
    mask: str = "none"              # 'none' | 'top_left' | 'bottom_right'
    window_left: int = -1
    window_right: int = 0
    num_sink: int = 0
    bias: Optional[str] = None      # None | 'alibi'
    sinks: bool = False             # per-head learnable sink logit
    seed: int = 0
    kv_chunks: int = 1              # >1: also run as K/V chunks joined by the lse merge
    notes: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.Dqk))

    @property
    def G(self) -> int:
        return self.Hq // self.Hk

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: sizes, dtypes and masks as stated for this operator.
WORKLOADS = {
    "mha_f32_s64": Workload(
        "mha_f32_s64", B=1, Hq=2, Hk=2, Sq=64, Sk=64, Dqk=64, Dv=64, dtype="f32",
        seed=1001, notes="MHA, fp32, no mask"),
    "gqa4_causal_tl_s1024": Workload(
        "gqa4_causal_tl_s1024", B=2, Hq=16, Hk=4, Sq=1024, Sk=1024, Dqk=128, Dv=128,
        dtype="bf16", mask="top_left", seed=1002, notes="GQA 4:1, top-left causal"),
    "gqa4_causal_br_s4096": Workload(
        "gqa4_causal_br_s4096", B=1, Hq=32, Hk=8, Sq=4096, Sk=4096, Dqk=128, Dv=128,
        dtype="bf16", mask="bottom_right", seed=1003, kv_chunks=4,
        notes="GQA 32:8, bottom-right causal, also as 4 K/V chunks of 1024"),
    "mha_alibi_dbias_s2048": Workload(
        "mha_alibi_dbias_s2048", B=4, Hq=16, Hk=16, Sq=2048, Sk=2048, Dqk=64, Dv=64,
        dtype="bf16", bias="alibi", seed=1004, notes="MHA + ALiBi bias, dbias summed over batch"),
    "gqa8_swa1024_sink4_s8192": Workload(
        "gqa8_swa1024_sink4_s8192", B=2, Hq=64, Hk=8, Sq=8192, Sk=8192, Dqk=128, Dv=128,
        dtype="bf16", mask="top_left", window_left=1023, window_right=0, num_sink=4,
        sinks=True, seed=1005, notes="GQA 8:1, window 1024 + 4 sink tokens + sink logit"),
}

# The configuration the throughput figure is quoted on.
HEADLINE = "gqa4_causal_br_s4096"


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def alibi_bias(H: int, Sq: int, Sk: int) -> np.ndarray:
    """[H, Sq, Sk] float32 ALiBi bias, shared over the batch."""
    slopes = np.array([2.0 ** (-(8.0 * (h + 1) / H)) for h in range(H)], dtype=np.float64)
    dist = np.abs(np.arange(Sq, dtype=np.float64)[:, None] - np.arange(Sk, dtype=np.float64)[None, :])
    out = np.empty((H, Sq, Sk), dtype=np.float32)
    for h in range(H):
        out[h] = (-slopes[h] * dist).astype(np.float32)
    return out


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw q, k, v, do (+ bias, sinks) for workload ``w`` as float32 arrays."""
    rng = np.random.default_rng(w.seed if seed is None else seed)

    def draw(shape):
        a = rng.standard_normal(shape).astype(np.float32)
        return round_bf16(a) if w.dtype == "bf16" else a

    out = {
        "q": draw((w.B, w.Hq, w.Sq, w.Dqk)),
        "k": draw((w.B, w.Hk, w.Sk, w.Dqk)),
        "v": draw((w.B, w.Hk, w.Sk, w.Dv)),
        "do": draw((w.B, w.Hq, w.Sq, w.Dv)),
        "bias": None,
        "sinks": None,
    }
    if w.sinks:
        out["sinks"] = rng.standard_normal(w.Hq).astype(np.float32)
    if w.bias == "alibi":
        out["bias"] = alibi_bias(w.Hq, w.Sq, w.Sk)
    return out


@dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch of sequences of different lengths (TND layout with
    cumulative sequence lengths).  Self-attention: each sequence's keys are
    its own rows.  Lengths are drawn uniformly from [min_len, max_len] with
    the seed, then rounded down to multiples of 8."""
    name: str
    n_seq: int
    min_len: int
    max_len: int
    Hq: int
    Hk: int
    D: int
    mask: str
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def lengths(self) -> np.ndarray:
        rng = np.random.default_rng(self.seed)
        return (rng.integers(self.min_len, self.max_len + 1, self.n_seq) // 8 * 8).astype(np.int64)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths())]).astype(np.int32)


VARLEN_WORKLOADS = {
    "varlen16_gqa4_causal_br": VarlenWorkload("varlen16_gqa4_causal_br", n_seq=16, min_len=256,
                                              max_len=4096, Hq=32, Hk=8, D=128, mask="bottom_right",
                                              seed=1006),
}


def make_varlen_inputs(w: VarlenWorkload) -> dict:
    """Packed q, do [T, Hq, D] and k, v [T, Hk, D] (bf16-rounded float32) and
    the prefix sums of the sequence lengths."""
    cu = w.cu_seqlens()
    T = int(cu[-1])
    rng = np.random.default_rng(w.seed + 1)
    draw = lambda *s: round_bf16(rng.standard_normal(s).astype(np.float32))
    return {"q": draw(T, w.Hq, w.D), "k": draw(T, w.Hk, w.D), "v": draw(T, w.Hk, w.D),
            "do": draw(T, w.Hq, w.D), "cu_seqlens": cu}


@dataclass(frozen=True)
class SharedKvWorkload:
    """Attention with one tensor as keys and values, head dim 512, in the
    packed TND layout of the CANN sparse_flash_mla_grad page ("Prototype",
    "Example": q and dO [T1, N1, D], kv [T2, N2, D], per-head sink logits,
    cumulative sequence lengths).  ``seqs`` lists each sequence's (query,
    key) lengths; the mask is a bottom-right sliding window of
    ``window_left + 1`` keys (the sliding-window case of that page)."""
    name: str
    seqs: tuple
    N1: int
    N2: int
    D: int
    window_left: int
    sinks: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def cu_seqlens(self):
        cu_q = np.concatenate([[0], np.cumsum([a for a, _ in self.seqs])]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum([b for _, b in self.seqs])]).astype(np.int32)
        return cu_q, cu_k

    @property
    def max_q(self) -> int:
        return max(a for a, _ in self.seqs)

    @property
    def max_k(self) -> int:
        return max(b for _, b in self.seqs)


SHARED_KV_WORKLOADS = {
    # the example's sizes: S1 = 256 queries, S2 = 1024 keys, N1 = 64, N2 = 1, D = 512
    "mla_swa512_s256x1024": SharedKvWorkload("mla_swa512_s256x1024", seqs=((256, 1024),), N1=64, N2=1,
                                             D=512, window_left=511, sinks=True, seed=1007),
    # one 4096-token sequence with the same heads
    "mla_swa512_s4096": SharedKvWorkload("mla_swa512_s4096", seqs=((4096, 4096),), N1=64, N2=1, D=512,
                                         window_left=511, sinks=True, seed=1008),
}


def make_shared_kv_inputs(w: SharedKvWorkload) -> dict:
    """Packed q, do [T1, N1, D], kv [T2, N2, D] (bf16-rounded float32), the
    sink logits [N1] and the prefix sums of the query and key lengths."""
    cu_q, cu_k = w.cu_seqlens()
    rng = np.random.default_rng(w.seed)
    draw = lambda *s: round_bf16(rng.standard_normal(s).astype(np.float32))  # noqa: E731
    out = {"q": draw(int(cu_q[-1]), w.N1, w.D), "kv": draw(int(cu_k[-1]), w.N2, w.D),
           "do": draw(int(cu_q[-1]), w.N1, w.D), "cu_q": cu_q, "cu_k": cu_k, "sinks": None}
    if w.sinks:
        out["sinks"] = rng.standard_normal(w.N1).astype(np.float32)
    return out
