"""Writes the small regression fixtures in this folder by calling only the
CPU oracle (``oracle/``).  The source pages print no numeric results for the
attention backward, so every stored value here comes from the oracle after
it has passed its pins (finite differences, library SDPA, invariants).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import MaskSpec, backward, forward  # noqa: E402

CASES = {
    # GQA 2:1, window 3 + 2 sink tokens + sink logit + bias, fp64 throughout
    "tiny_gqa_window_sink_bias": dict(B=1, Hq=2, Hk=1, Sq=5, Sk=6, D=3, seed=2024,
                                      spec=dict(kind="bottom_right", window_left=2, window_right=0, num_sink=2),
                                      bias=True, sinks=True, scale=0.5),
    # plain causal MHA
    "tiny_mha_causal": dict(B=1, Hq=2, Hk=2, Sq=4, Sk=4, D=2, seed=7,
                            spec=dict(kind="top_left"), bias=False, sinks=False, scale=0.7),
}


def build(c):
    rng = np.random.default_rng(c["seed"])
    q = rng.standard_normal((c["B"], c["Hq"], c["Sq"], c["D"]))
    k = rng.standard_normal((c["B"], c["Hk"], c["Sk"], c["D"]))
    v = rng.standard_normal((c["B"], c["Hk"], c["Sk"], c["D"]))
    do = rng.standard_normal((c["B"], c["Hq"], c["Sq"], c["D"]))
    bias = rng.standard_normal((c["Hq"], c["Sq"], c["Sk"])) if c["bias"] else None
    sinks = rng.standard_normal(c["Hq"]) if c["sinks"] else None
    return q, k, v, do, bias, sinks


def main():
    for name, c in CASES.items():
        q, k, v, do, bias, sinks = build(c)
        spec = MaskSpec(**c["spec"])
        o, lse = forward(q, k, v, c["scale"], spec, bias, sinks)
        g = backward(q, k, v, o, do, lse, c["scale"], spec, bias, sinks)
        out = {"case": c, "source": "oracle/ (fp64) -- the pages print no values",
               "o": o.tolist(), "lse": lse.tolist()}
        for key in ("dq", "dk", "dv", "dbias", "dsinks"):
            out[key] = None if g[key] is None else g[key].tolist()
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
