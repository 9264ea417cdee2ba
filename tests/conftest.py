import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_sessionfinish(session, exitstatus):
    """Write the per-workload parity counts (rows, exact, tolerated by class,
    value checks, failures) gathered by the GPU parity tests to the file
    named by SPECV_PARITY_RECORD, when set."""
    path = os.environ.get("SPECV_PARITY_RECORD")
    if not path:
        return
    try:
        from parity import RECORDS
    except ImportError:
        return
    if not RECORDS:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"exit_status": int(exitstatus), "workloads": RECORDS}, f, indent=1, sort_keys=True)
