"""Pins for the oracle's mask predicate and pair counts.

Each reference mask below is written as plain loops straight from the
definitions on the pages, independent of ``oracle.allowed_mask``:
  * CK FMHA example 22 "Sink Token Attention FMHA": make_causal_mask (j <= i),
    make_causal_sink_mask (j < num_sink or j <= i),
    make_sliding_window_sink_mask (j < num_sink or i - W + 1 <= j <= i);
  * CANN sparse_flash_mla_grad "Example": bottom-right rows may use keys
    below threshold = (S2 - S1) + s1 + 1.
"""
import numpy as np
import pytest

from oracle import MaskSpec, allowed_mask, allowed_pair_count
from attention_backward_attn_amd import mask as hostmask


def dense(sq, sk, spec):
    return allowed_mask(np.arange(sq)[:, None], np.arange(sk)[None, :], sq, sk, spec)


def loops(sq, sk, pred):
    out = np.zeros((sq, sk), dtype=bool)
    for i in range(sq):
        for j in range(sk):
            out[i, j] = pred(i, j)
    return out


@pytest.mark.parametrize("sq,sk", [(7, 7), (16, 16), (5, 9)])
def test_top_left_causal(sq, sk):
    ref = loops(sq, sk, lambda i, j: j <= i)
    assert np.array_equal(dense(sq, sk, MaskSpec("top_left")), ref)


@pytest.mark.parametrize("ns", [0, 1, 2, 4, 8])
def test_causal_sink(ns):
    ref = loops(20, 20, lambda i, j: j < ns or j <= i)
    assert np.array_equal(dense(20, 20, MaskSpec("top_left", num_sink=ns)), ref)


@pytest.mark.parametrize("w,ns", [(4, 2), (8, 4), (1, 0), (3, 0), (64, 4)])
def test_window_sink(w, ns):
    ref = loops(24, 24, lambda i, j: j < ns or (i - w + 1 <= j <= i))
    got = dense(24, 24, MaskSpec("top_left", window_left=w - 1, window_right=0, num_sink=ns))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("sq,sk", [(4, 10), (10, 10), (10, 4), (1, 7)])
def test_bottom_right_threshold(sq, sk):
    delta_s = sk - sq

    def pred(i, j):
        threshold = delta_s + i + 1 if delta_s + i + 1 >= 0 else 0
        return j < threshold

    assert np.array_equal(dense(sq, sk, MaskSpec("bottom_right")), loops(sq, sk, pred))


def test_sinks_zero_is_causal():
    a = dense(33, 33, MaskSpec("top_left", num_sink=0))
    b = dense(33, 33, MaskSpec("top_left"))
    assert np.array_equal(a, b)


def test_none_is_dense():
    assert dense(5, 6, MaskSpec("none")).all()


def test_offsets_match_slices():
    """A chunk with global offsets sees exactly the slice of the full mask."""
    full = dense(40, 48, MaskSpec("bottom_right", window_left=9, num_sink=3))
    for q0, k0, sq, sk in [(0, 0, 40, 12), (0, 12, 40, 12), (8, 24, 16, 24), (30, 36, 10, 12)]:
        spec = MaskSpec("bottom_right", window_left=9, num_sink=3, q_offset=q0, k_offset=k0,
                        sq_total=40, sk_total=48)
        assert np.array_equal(dense(sq, sk, spec), full[q0:q0 + sq, k0:k0 + sk])


def test_pair_counts_small_closed_forms():
    n = 64
    assert allowed_pair_count(n, n, MaskSpec("top_left")) == n * (n + 1) // 2
    assert allowed_pair_count(n, n, MaskSpec("none")) == n * n
    # window W, no sinks: rows i < W see i + 1 keys, the rest see W
    W = 16
    assert allowed_pair_count(n, n, MaskSpec("top_left", window_left=W - 1)) == \
        W * (W + 1) // 2 + (n - W) * W


SPECS = [
    (64, 64, MaskSpec("none")),
    (64, 64, MaskSpec("top_left")),
    (48, 80, MaskSpec("bottom_right")),
    (80, 48, MaskSpec("bottom_right")),
    (100, 100, MaskSpec("top_left", window_left=15, num_sink=4)),
    (100, 100, MaskSpec("top_left", window_left=0, num_sink=1)),
    (64, 96, MaskSpec("bottom_right", window_left=7, window_right=3, num_sink=2)),
    (37, 53, MaskSpec("top_left", window_left=5, window_right=2, num_sink=3, q_offset=11,
                      k_offset=7, sq_total=90, sk_total=120)),
]


@pytest.mark.parametrize("sq,sk,spec", SPECS)
def test_host_pair_count_matches_oracle(sq, sk, spec):
    """The host-side closed-form pair counter (used for the FLOP figure)
    equals the oracle's brute-force count."""
    assert hostmask.allowed_pairs(sq, sk, spec.kind, spec.window_left, spec.window_right,
                                  spec.num_sink, spec.q_offset, spec.k_offset,
                                  spec.sq_total, spec.sk_total) == allowed_pair_count(sq, sk, spec)


@pytest.mark.slow
@pytest.mark.parametrize("name,expected", [
    ("gqa4_causal_tl_s1024", 524800),
    ("gqa4_causal_br_s4096", 8390656),
    ("gqa8_swa1024_sink4_s8192", 7893504),
])
def test_workload_pair_counts(name, expected):
    from attention_backward_attn_amd.inputs import WORKLOADS
    w = WORKLOADS[name]
    spec = MaskSpec(w.mask, w.window_left, w.window_right, w.num_sink)
    # closed forms: causal n(n+1)/2; window W + sinks: see test above, plus
    # sink keys outside the window
    assert allowed_pair_count(w.Sq, w.Sk, spec) == expected
    assert hostmask.allowed_pairs(w.Sq, w.Sk, w.mask, w.window_left, w.window_right,
                                  w.num_sink) == expected
