"""Full-size fp64 oracle references for the GPU parity tests, computed in
parallel over independent units of work.

Attention splits exactly into (batch entry b, KV head g) units: the query
heads of group g in entry b read only K/V of (b, g), their dQ rows and the
group's dK/dV depend on nothing else, and only dbias (summed over the
batch, per query head) and dsinks (summed over batch and rows) collect
across units.  Each unit runs the oracle as it stands -- ``oracle.forward``,
its O / LSE rounded to fp32 (the buffers the GPU backward also receives),
then ``oracle.backward`` -- on that unit's slices; the parent stitches the
slices together and adds the dbias / dsinks contributions of the batch
entries in batch order.  No arithmetic of the method happens here.

The worker processes are forked once per test session, before any test
touches the GPU (tests/conftest.py starts the pool when a selected test is
marked ``full_oracle``), and each runs single-threaded BLAS.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import sys
import time

import numpy as np

_POOL = None
_CACHE: dict = {}


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def start(n: int | None = None):
    """Fork the worker pool (call before the GPU is initialised)."""
    global _POOL
    if _POOL is None:
        n = n or max(1, min(16, os.cpu_count() or 1))
        _POOL = mp.get_context("fork").Pool(n, initializer=_init_worker)
    return _POOL


def stop():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None
    _CACHE.clear()


def _unit(args):
    """Forward (fp32 O / LSE) and backward of one (b, g) unit."""
    import oracle
    q, k, v, do, bias, sinks, scale, spec = args
    o64, l64 = oracle.forward(q, k, v, scale, spec, bias, sinks, row_block=1024)
    o32, l32 = o64.astype(np.float32), l64.astype(np.float32)
    g = oracle.backward(q, k, v, o32, do, l32, scale, spec, bias, sinks, row_block=1024)
    return {"o": o32, "lse": l32, "o64": o64, **g}


def reference(name: str, w, x, spec, say=print) -> dict:
    """Oracle O, LSE (fp32 and fp64 O) and dq, dk, dv, dbias, dsinks, delta
    of workload ``w`` on inputs ``x`` (cached per workload name)."""
    if name in _CACHE:
        return _CACHE[name]
    pool = _POOL if _POOL is not None else start()
    G = w.G
    units = [(b, g) for b in range(w.B) for g in range(w.Hk)]

    def args(b, g):
        hs = slice(g * G, (g + 1) * G)
        return (x["q"][b:b + 1, hs], x["k"][b:b + 1, g:g + 1], x["v"][b:b + 1, g:g + 1], x["do"][b:b + 1, hs],
                None if x["bias"] is None else x["bias"][hs], None if x["sinks"] is None else x["sinks"][hs],
                w.scale, spec)

    t0 = time.perf_counter()
    ref = {"o": np.empty((w.B, w.Hq, w.Sq, w.Dv), np.float32), "lse": np.empty((w.B, w.Hq, w.Sq), np.float32),
           "o64": np.empty((w.B, w.Hq, w.Sq, w.Dv)), "dq": np.empty((w.B, w.Hq, w.Sq, w.Dqk)),
           "dk": np.empty((w.B, w.Hk, w.Sk, w.Dqk)), "dv": np.empty((w.B, w.Hk, w.Sk, w.Dv)),
           "delta": np.empty((w.B, w.Hq, w.Sq)),
           "dbias": None if x["bias"] is None else np.zeros((w.Hq, w.Sq, w.Sk)),
           "dsinks": None if x["sinks"] is None else np.zeros(w.Hq)}
    done = 0
    # imap keeps unit order: batch entries arrive in order, so the dbias /
    # dsinks sums over the batch are taken in a fixed order
    for (b, g), r in zip(units, pool.imap(_unit, (args(b, g) for b, g in units))):
        hs = slice(g * G, (g + 1) * G)
        for key in ("o", "lse", "o64", "dq", "delta"):
            ref[key][b, hs] = r[key][0]
        ref["dk"][b, g] = r["dk"][0, 0]
        ref["dv"][b, g] = r["dv"][0, 0]
        if ref["dbias"] is not None:
            ref["dbias"][hs] += r["dbias"]
        if ref["dsinks"] is not None:
            ref["dsinks"][hs] += r["dsinks"]
        done += 1
        if done % max(1, len(units) // 4) == 0 or done == len(units):
            say(f"  oracle {name}: {done}/{len(units)} units, {time.perf_counter() - t0:.1f} s")
            sys.stdout.flush()
    _CACHE[name] = ref
    return ref


def drop(name: str):
    _CACHE.pop(name, None)
