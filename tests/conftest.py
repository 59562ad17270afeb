import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (minutes of CPU work)")


def pytest_terminal_summary(terminalreporter):
    """Near-ties are reported, never forgiven silently: every position where
    the oracle's top-2 margin was below 1e-3 (or a probe logit sat within the
    gate's tolerance of the threshold), whichever test met it."""
    try:
        from parity import NEAR_TIES
    except Exception:  # pragma: no cover
        return
    ids = [r for r in NEAR_TIES if r["kind"] == "drafted id"]
    gates = [r for r in NEAR_TIES if r["kind"] == "probe gate"]
    terminalreporter.write_line(f"near-ties: {len(ids)} drafted-id positions with an oracle top-2 margin below 1e-3, "
                                f"{len(gates)} probe rows within the gate tolerance of the threshold")
    for r in NEAR_TIES[:50]:
        terminalreporter.write_line(f"  {r}")
    path = os.environ.get("DSPARK_NEAR_TIES_JSON")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(NEAR_TIES, f, indent=1, default=float)
