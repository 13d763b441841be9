#!/usr/bin/env python3
"""Attention-backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole backward of the workload on inputs already resident in
HBM: ``attn_bwd_preprocess`` (delta = rowsum(dO * O)) followed by
``attn_bwd`` (the dK / dV pass by key blocks, then the dQ pass by query
blocks), writing dQ, dK, dV.  O and LSE come from the library's own forward
before the timed region.  Throughput counts
2 * (3 * Dqk + 2 * Dv) FLOPs per allowed (query, key) pair per query head --
the five contractions -- and nothing for masked pairs or recomputation.

Before the W warmup steps the step runs untimed for ``--settle-ms``
(default 500 ms) so that the timed steps see the GPU's steady clock.

Rank 0 prints one JSON line.  It also carries
  * ``roofline`` for the main backward call (``attn_bwd``: its two kernels,
    timed together with HIP events on the stream they run on; the
    rocprofv3 summary lists each),
  * ``cpu_baseline``: the fp64 CPU oracle timed on a bounded sample of the
    same workload (a subset of the KV head groups),
  * extra timings (deterministic mode, the 4-chunk K/V split with the lse
    merge, the forward, a packed variable-length batch, and the shared-KV
    head-dim-512 path).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed load before the warmup steps, to reach the steady GPU clock")
    ap.add_argument("--workload", default=None, help="workload name (default: the headline workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip deterministic / chunked / forward timings")
    ap.add_argument("--cpu-groups", type=int, default=8, help="KV head groups in the CPU oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (HBM counter calibration)")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter
    readings calibrate the counters of the attention kernels."""
    import torch
    n = 256 * 1024 * 1024 // 4
    src = torch.ones(n, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4, "launches": 3}))


def traffic_record(kernel_key: str):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
        from attention_backward_attn_amd.build import source_digest
        if rec and rec.get("source_digest") == source_digest():
            return rec.get("bytes_per_launch")
    except Exception:
        return None
    return None


def roofline(w, flops: float, main_ms: float, main_med: float, traffic) -> dict:
    """Roofline of the attn_bwd call.  The ALiBi + dbias workload (fp32 bias
    and dbias of [Hq, Sq, Sk] dominate its bytes) is bound by HBM: achieved =
    algorithmic bytes / time against 8 TB/s.  The fp32 workload runs on the
    vector ALU (fp32 FMA peak).  The others are bound by the bf16 matrix
    cores: achieved = counted FLOPs / time."""
    from attention_backward_attn_amd.mask import backward_bytes
    out = {"kernel": "attn_bwd (k_dkdv3/k_dkdv2/k_dkdv + k_dq2/k_dq/k_dqb)" if w.dtype == "bf16" else
           "attn_bwd (k_dkdv_simt + k_dq_simt)", "kernel_ms_mean": round(main_ms, 4),
           "kernel_ms_median": round(main_med, 4), "algorithmic_bytes": backward_bytes(w)}
    if w.bias:
        gbs = backward_bytes(w) / (main_ms * 1e-3) / 1e9
        out.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_GBS, 4), "traffic": traffic})
        out["mfma_tflops"] = round(flops / (main_ms * 1e-3) / 1e12, 2)
    else:
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = flops / (main_ms * 1e-3) / 1e12
        out.update({"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(achieved, 2),
                    "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic})
    return {k: out[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")} | \
        {k: v for k, v in out.items() if k not in ("bound", "achieved", "peak", "unit", "frac", "traffic")}


def bench_varlen(stream, name: str = "varlen16_gqa4_causal_br", steps: int = 10):
    """Backward of a packed variable-length batch (TND with cumulative
    sequence lengths): preprocess + attn_bwd per step, counted FLOPs summed
    over the sequences."""
    import numpy as np
    import torch

    from attention_backward_attn_amd import binding as ab
    from attention_backward_attn_amd.inputs import VARLEN_WORKLOADS, make_varlen_inputs
    from attention_backward_attn_amd.mask import allowed_pairs
    w = VARLEN_WORKLOADS[name]
    x = make_varlen_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(x[n]).to(dev, torch.bfloat16) for n in ("q", "k", "v", "do"))
    cu = torch.from_numpy(x["cu_seqlens"]).to(dev)
    lens = np.diff(x["cu_seqlens"])
    kw = dict(mask=w.mask, cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=int(lens.max()),
              max_seqlen_k=int(lens.max()))
    o, lse = ab.forward(q, k, v, scale=w.scale, stream=stream, **kw)
    dq = torch.empty(q.shape, device=dev)
    dk = torch.empty(k.shape, device=dev)
    dv = torch.empty(v.shape, device=dev)
    delta = torch.empty(lse.shape, device=dev)
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, scale=w.scale, **kw)

    def step():
        ab.attn_bwd_preprocess(p, o, do, lse, None, delta, None, None, None, None, stream)
        ab.attn_bwd(p, q, k, v, do, lse, delta, None, dq, dk, dv, None, 0, stream)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = sum(allowed_pairs(int(n), int(n), w.mask) for n in lens)
    flops = 10.0 * w.D * pairs * w.Hq
    return {"workload": name, "tokens": int(lens.sum()), "n_seq": int(len(lens)), "ms_per_step": round(ms, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}


def bench_shared_kv(stream, name: str = "mla_swa512_s4096", steps: int = 10, warmup: int = 3) -> dict:
    """One tensor as keys and values at head dim 512 (packed TND, bottom-right
    sliding window, sink logits): preprocess + attn_bwd with ATTN_SHARED_KV
    per step, and the forward.  Counted FLOPs as for the other workloads,
    10 * D per allowed pair per query head (dK and dV of the shared tensor
    are both counted; they are both computed)."""
    import numpy as np
    import torch

    from attention_backward_attn_amd import binding as ab
    from attention_backward_attn_amd.inputs import SHARED_KV_WORKLOADS, make_shared_kv_inputs
    from attention_backward_attn_amd.mask import allowed_pairs
    w = SHARED_KV_WORKLOADS[name]
    x = make_shared_kv_inputs(w)
    dev = torch.device("cuda:0")
    q, kv, do = (torch.from_numpy(x[n]).to(dev, torch.bfloat16) for n in ("q", "kv", "do"))
    sinks = None if x["sinks"] is None else torch.from_numpy(x["sinks"]).to(dev)
    kw = dict(mask="bottom_right", window_left=w.window_left, cu_seqlens_q=torch.from_numpy(x["cu_q"]).to(dev),
              cu_seqlens_k=torch.from_numpy(x["cu_k"]).to(dev), max_seqlen_q=w.max_q, max_seqlen_k=w.max_k)
    # O in the inputs' dtype (the page requires attn_out to match q)
    o, lse = ab.forward(q, kv, kv, sinks=sinks, scale=w.scale, o_dtype=torch.bfloat16, stream=stream, **kw)
    dq = torch.empty(q.shape, device=dev)
    dkv = torch.empty(kv.shape, device=dev)
    delta = torch.empty(lse.shape, device=dev)
    dsinks = torch.empty(w.N1, device=dev) if sinks is not None else None
    p = ab.make_problem(q, kv, kv, o=o, do=do, dq=dq, dk=dkv, scale=w.scale, **kw)
    # caller-owned workspace for the query-head parts' partial sums
    ws = ab.set_workspace(p, ab.ATTN_SHARED_KV)  # noqa: F841

    def step():
        ab.attn_bwd_preprocess(p, o, do, lse, sinks, delta, dsinks, None, None, None, stream)
        ab.attn_bwd(p, q, kv, kv, do, lse, delta, None, dq, dkv, None, None, ab.ATTN_SHARED_KV, stream)

    def fwd():
        ab.attn_fwd_lse(p, q, kv, kv, None, sinks, o, lse, stream)

    def time_it(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    ms = time_it(step, steps)
    fwd_ms = time_it(fwd, steps)
    pairs = sum(allowed_pairs(a, b, "bottom_right", w.window_left) for a, b in w.seqs)
    flops = 10.0 * w.D * pairs * w.N1
    return {"workload": name, "T1": int(x["cu_q"][-1]), "T2": int(x["cu_k"][-1]), "N1": w.N1, "N2": w.N2,
            "D": w.D, "window_left": w.window_left, "allowed_pairs_per_head": pairs, "counted_flop": flops,
            "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "pct_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "forward_ms": round(fwd_ms, 4),
            "forward_tflops": round(4.0 * w.D * pairs * w.N1 / (fwd_ms * 1e-3) / 1e12, 2)}


def cpu_baseline(w, x, groups: int):
    """Time the fp64 oracle backward on KV groups [0, groups) of batch 0."""
    import numpy as np

    import oracle
    from attention_backward_attn_amd.mask import backward_flops
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count()
    groups = max(1, min(groups, w.Hk))
    heads = slice(0, groups * w.G)
    spec = oracle.MaskSpec(w.mask, w.window_left, w.window_right, w.num_sink)
    q, do = x["q"][:1, heads], x["do"][:1, heads]
    k, v = x["k"][:1, :groups], x["v"][:1, :groups]
    bias = None if x["bias"] is None else x["bias"][heads]
    sinks = None if x["sinks"] is None else x["sinks"][heads]
    o, lse = oracle.forward(q, k, v, w.scale, spec, bias, sinks, row_block=1024)
    o, lse = o.astype(np.float32), lse.astype(np.float32)
    t0 = time.perf_counter()
    oracle.backward(q, k, v, o, do, lse, w.scale, spec, bias, sinks, row_block=1024)
    dt = time.perf_counter() - t0
    flops = backward_flops(w.with_(B=1, Hq=groups * w.G, Hk=groups))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle backward (no forward), batch 0, KV groups 0..{groups - 1} "
                      f"({groups * w.G} of {w.Hq} query heads), {dt:.2f} s; host cpu_count={os.cpu_count()}",
            "seconds": dt}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from attention_backward_attn_amd import binding as ab
    from attention_backward_attn_amd.inputs import HEADLINE, WORKLOADS, make_inputs
    from attention_backward_attn_amd.mask import allowed_pairs, backward_flops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from attention_backward_attn_amd.inputs import SHARED_KV_WORKLOADS
    if args.workload in SHARED_KV_WORKLOADS:
        # the shared-KV (head dim 512) path alone, on its own line
        r = bench_shared_kv(torch.cuda.current_stream(), args.workload, steps=args.steps, warmup=args.warmup)
        print(json.dumps({"metric": "shared-KV attention-backward TFLOP/s (D=512)", "value": r["tflops"],
                          "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
                          "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) inputs)",
                          "config": {"workload": args.workload}, "shared_kv": r}), flush=True)
        return
    w = WORKLOADS[args.workload or HEADLINE]
    dev = torch.device("cuda:0")
    x = make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def todev(a, t):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, t)

    q, k, v, do = (todev(x[n], dt) for n in ("q", "k", "v", "do"))
    bias, sinks = todev(x["bias"], torch.float32), todev(x["sinks"], torch.float32)
    mask_kw = dict(mask=w.mask, window_left=w.window_left, window_right=w.window_right,
                   num_sink_tokens=w.num_sink)
    stream = torch.cuda.current_stream()
    o, lse = ab.forward(q, k, v, bias=bias, sinks=sinks, scale=w.scale, stream=stream, **mask_kw)
    dq = torch.empty(q.shape, device=dev, dtype=torch.float32)
    dk = torch.empty(k.shape, device=dev, dtype=torch.float32)
    dv = torch.empty(v.shape, device=dev, dtype=torch.float32)
    delta = torch.empty(lse.shape, device=dev, dtype=torch.float32)
    dsinks = torch.empty(w.Hq, device=dev, dtype=torch.float32) if sinks is not None else None
    dbias = torch.empty(bias.shape, device=dev, dtype=torch.float32) if bias is not None else None
    p = ab.make_problem(q, k, v, o=o, do=do, dq=dq, dk=dk, dv=dv, bias=bias, scale=w.scale, **mask_kw)
    # caller-owned workspace for split key blocks' partial sums (none when
    # the call needs none), allocated before any timing
    ws = ab.set_workspace(p, 0, bias=bias)  # noqa: F841

    def pre():
        ab.attn_bwd_preprocess(p, o, do, lse, sinks, delta, dsinks, None, None, None, stream)

    def main(flags):
        # attn_bwd overwrites dQ, dK, dV (and dbias); it zeroes by itself
        # whatever its split parts add into.
        ab.attn_bwd(p, q, k, v, do, lse, delta, bias, dq, dk, dv, dbias, flags, stream)

    def step(flags):
        pre()
        main(flags)

    def region(fn, n):
        """Mean ms of n back-to-back calls of fn on the bench stream, between
        two HIP events on that stream (no event between the calls: a
        recorded event costs the stream several microseconds)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def timed(flags, steps, warmup):
        """The timed region: exactly `steps` steps between a synchronize and
        a HIP event on each side; then the two calls of a step on their own
        (back-to-back regions of the same length) for the per-call times."""
        for _ in range(warmup):
            step(flags)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        span = region(lambda: step(flags), steps)
        wall = time.perf_counter() - t0
        pre_ms = region(pre, steps)
        # attn_bwd alone: the mean over one region, the median of five shorter ones
        main_ms = region(lambda: main(flags), steps)
        n5 = max(1, steps // 5)
        subs = [region(lambda: main(flags), n5) for _ in range(5)]
        return wall * 1e3 / steps, span, pre_ms, main_ms, float(np.median(subs))

    flops = backward_flops(w)
    pairs = allowed_pairs(w.Sq, w.Sk, w.mask, w.window_left, w.window_right, w.num_sink)
    # Clock settle: the GPU takes a few hundred milliseconds of load to reach
    # its steady clock; run the step (untimed) for that long before the
    # warmup steps, so the timed steps see the steady state.
    def settle(flags, ms):
        t_end = time.perf_counter() + ms * 1e-3
        n = 0
        while time.perf_counter() < t_end:
            step(flags)
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return n

    n_settle = settle(0, args.settle_ms)
    wall_ms, span_ms, pre_ms, main_ms, main_med = timed(0, args.steps, args.warmup)
    ms_per_step = span_ms
    value = flops / (ms_per_step * 1e-3) / 1e12
    kernel_key = f"bwd_main:{w.name}"
    out = {
        "metric": ("attention-backward TFLOP/s + % bf16 MFMA peak (GQA 32:8, S=4096, D=128, causal)"
                   if w.name == HEADLINE else f"attention-backward TFLOP/s + % bf16 MFMA peak ({w.name})"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs; O/LSE from the library forward)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hk": w.Hk, "Sq": w.Sq, "Sk": w.Sk,
                   "D": w.Dqk, "mask": w.mask, "window_left": w.window_left, "num_sink": w.num_sink,
                   "bias": w.bias, "sinks": w.sinks, "allowed_pairs_per_head": pairs,
                   "counted_flop": flops, "timed": "attn_bwd_preprocess + attn_bwd (dK/dV pass + dQ pass)"},
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "wall_ms_per_step": round(wall_ms, 4),
        "preprocess_ms": round(pre_ms, 4),
        "clock_settle": {"ms": args.settle_ms, "steps": n_settle},
        "roofline": roofline(w, flops, main_ms, main_med, traffic_record(kernel_key)),
    }
    if not args.no_extras:
        # (its own clock settle and as many steps as the headline line)
        settle(ab.ATTN_DETERMINISTIC, min(args.settle_ms, 200.0))
        _, span_d, _, main_d, _ = timed(ab.ATTN_DETERMINISTIC, args.steps, args.warmup)
        out["deterministic"] = {"ms_per_step": round(span_d, 4),
                                "tflops": round(flops / (span_d * 1e-3) / 1e12, 2)}
        # forward (input producer), timed for context: attn_fwd_lse into
        # buffers of its own, warmed up, then a region of back-to-back calls
        o_f, lse_f = torch.empty_like(o), torch.empty_like(lse)

        def fwd():
            ab.attn_fwd_lse(p, q, k, v, bias, sinks, o_f, lse_f, stream)
        for _ in range(3):
            fwd()
        fwd_ms = region(fwd, args.steps)
        out["forward"] = {"ms": round(fwd_ms, 4),
                          "tflops": round(2 * (w.Dqk + w.Dv) * pairs * w.B * w.Hq / (fwd_ms * 1e-3) / 1e12, 2)}
        if w.kv_chunks > 1 and bias is None and sinks is None:
            n, c = w.kv_chunks, w.Sk // w.kv_chunks
            probs = [ab.make_problem(q, k[:, :, i * c:(i + 1) * c], v[:, :, i * c:(i + 1) * c], o=o, do=do, dq=dq,
                                     dk=dk[:, :, i * c:(i + 1) * c], dv=dv[:, :, i * c:(i + 1) * c], scale=w.scale,
                                     k_offset=i * c, sk_total=w.Sk, **mask_kw) for i in range(n)]
            # the first chunk writes dQ, the others add to it (the same sum as
            # zeroed dQ plus every chunk, without the zero fill and one read)
            fl_c = [0] + [ab.ATTN_ACCUMULATE_DQ] * (n - 1)
            ws_c = [ab.set_workspace(pc, f) for pc, f in zip(probs, fl_c)]  # noqa: F841

            def chunked():
                ab.attn_bwd_preprocess(p, o, do, lse, None, delta, None, None, None, None, stream)
                for i in range(n):
                    sl = slice(i * c, (i + 1) * c)
                    ab.attn_bwd(probs[i], q, k[:, :, sl], v[:, :, sl], do, lse, delta, None, dq, dk[:, :, sl],
                                dv[:, :, sl], None, fl_c[i], stream)
            for _ in range(2):
                chunked()
            ch_ms = region(chunked, 5)
            out["chunked_kv4"] = {"ms_per_step": round(ch_ms, 4), "tflops": round(flops / (ch_ms * 1e-3) / 1e12, 2)}
        if w.name == HEADLINE:
            out["varlen"] = bench_varlen(stream)
            out["shared_kv"] = bench_shared_kv(stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_groups)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
