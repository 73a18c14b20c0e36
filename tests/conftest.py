import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import json

import pytest


@pytest.fixture(autouse=True)
def _parity_error_report(request):
    """After each test: the largest |gpu - ref| / ||chunk|| per output kind that the parity
    comparisons saw (printed; appended as a JSON line to $PARITY_STATS_FILE if set)."""
    parity = sys.modules.get("parity")
    if parity is not None:
        parity.STATS.clear()
    yield
    parity = sys.modules.get("parity")
    if parity is None or not parity.STATS:
        return
    stats = {k: float(v) for k, v in parity.STATS.items()}
    print(f"\n[parity max |gpu-ref|/||chunk||] {request.node.nodeid}: " +
          ", ".join(f"{k} {v:.3e}" for k, v in sorted(stats.items())), flush=True)
    path = os.environ.get("PARITY_STATS_FILE")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": request.node.nodeid, **stats}) + "\n")
