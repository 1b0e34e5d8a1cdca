import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """With TP_PARITY_REPORT set, write every parity comparison of the run
    (per-tensor, per-block and element-wise errors) to that file, one JSON
    object per case."""
    path = os.environ.get("TP_PARITY_REPORT")
    if not path:
        return
    try:
        from tests import gpu_harness
    except Exception:
        return
    if not gpu_harness.REPORT:
        return
    import json
    with open(path, "w") as f:
        for rec in gpu_harness.REPORT:
            f.write(json.dumps(rec) + "\n")
