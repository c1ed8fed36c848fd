import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionfinish(session, exitstatus):
    """With RSWA_PARITY_LOG set, write the observed error maxima of every
    GPU parity comparison (gpu_harness.compare) to that JSON file."""
    path = os.environ.get("RSWA_PARITY_LOG")
    if not path:
        return
    import json

    gh = sys.modules.get("gpu_harness")
    if gh is None or not gh.ERROR_LOG:
        return
    recs = [{"test": t, "output": k, "dtype": d, **v} for (t, k, d), v in sorted(gh.ERROR_LOG.items())]
    with open(path, "w") as f:
        json.dump(recs, f, indent=1)
