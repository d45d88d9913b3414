import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for _p in (HERE, ROOT):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU oracle runs")
    # the oracle's worker processes must be forked from a process that has
    # not touched the GPU: fork them before any test runs
    import oracle_pool
    oracle_pool.start()


def pytest_unconfigure(config):
    import oracle_pool
    oracle_pool.shutdown()


def read_golden(name):
    """key -> int from a tests/golden text fixture (comment lines start with #)."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            out[k] = int(v)
    return out
