import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
    config.addinivalue_line("markers", "full_oracle: compares with the oracle on a full-size workload "
                                       "(references computed by the forked worker pool of oracle_pool)")


def pytest_collection_finish(session):
    # Fork the oracle worker pool now, before any test initialises the GPU:
    # the workers then inherit no GPU state.
    if any(item.get_closest_marker("full_oracle") for item in session.items):
        import oracle_pool
        oracle_pool.start()


def pytest_sessionfinish(session, exitstatus):
    mod = sys.modules.get("oracle_pool")
    if mod is not None:
        mod.stop()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    mod = sys.modules.get("parity_util")
    if mod is None or not mod.MARGINS:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity margins: max|gpu - ref| / max|ref| (abs: zero reference) against the bound")
    worst = {}
    for test, name, val, bound, kind in mod.MARGINS:
        key = (test, name, kind)
        if key not in worst or val / bound > worst[key][0] / worst[key][1]:
            worst[key] = (val, bound)
    for (test, name, kind), (val, bound) in worst.items():
        tr.write_line(f"{test:60s} {name:28s} {kind} {val:.3e} <= {bound:g}  ({100 * val / bound:5.1f}% of bound)")
