"""Plain fp64 CPU oracle for the fused attention backward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers or
constants): every function is written out from the defining formulas on the
source pages, in fp64, with no blocking or fusion beyond restricting each row
block to the key columns that can carry probability mass.

Sources (cited by page title and section throughout):

* [GQA-BWD]  CK FMHA dispatcher example 34, "Backward Pass with GQA"
  (``34_bwd_gqa_fmha.py``): the CPU backward reference in the module docstring
  and ``cpu_bwd_gqa``; the forward with intermediates
  ``cpu_fwd_with_intermediates``; the GQA == expanded-MHA equivalence check.
* [DBIAS]    CK FMHA dispatcher example 28, "Backward Bias Gradient (dbias)
  FMHA" (``28_backward_dbias_fmha.py``): ``make_alibi_bias``,
  ``cpu_attention_fwd_bias``, ``cpu_attention_bwd_dbias``, the finite-difference
  gradient verification (Step 4).
* [SFMG]     CANN ops-transformer ``sparse_flash_mla_grad`` operator page:
  "Formula" (Phase 2: P, dP, dS; Phase 3: dQ, dKV, dSinks), "Prototype",
  "Constraints", and the bottom-right ``threshold`` rule in "Example".
* [SINK]     CK FMHA dispatcher example 22, "Sink Token Attention FMHA"
  (``22_sink_tokens_fmha.py``): ``make_causal_mask``,
  ``make_causal_sink_mask``, ``make_sliding_window_sink_mask``,
  ``cpu_attention_fwd_masked``.
* [RING]     "Ring attention for PyTorch" gist (``ring_attn.py``):
  ``_ring_fwd`` (log-sum-exp merge of partial (o, lse)), ``_ring_bwd``
  (per-chunk backward against the global o and lse).

Parity status of each function is listed in ``oracle/attention.py``'s header.
"""

from .attention import (  # noqa: F401
    MaskSpec,
    allowed_mask,
    forward,
    preprocess,
    backward,
    lse_merge,
    dq_rows,
    dkdv_keys,
    ds_rows,
    allowed_pair_count,
    forward_varlen,
    backward_varlen,
    backward_shared_kv,
    backward_shared_kv_varlen,
)
