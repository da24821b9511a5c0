import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _gpu_runtime_first(request):
    """In a session that runs GPU tests, bring up the GPU runtime before any
    test starts worker threads (the input generators use a thread pool)."""
    if any(item.get_closest_marker("gpu") for item in request.session.items):
        import torch
        if torch.cuda.is_available():
            torch.cuda.init()
            torch.zeros(1, device="cuda")
    yield


@pytest.fixture(scope="session")
def golden():
    import json

    def load(name):
        with open(os.path.join(ROOT, "tests", "golden", name)) as f:
            return json.load(f)
    return load


def pytest_terminal_summary(terminalreporter):
    """Max errors of the GPU parity runs against their tolerances, so that a
    quiet (-q) run still shows each workload's margin."""
    gu = sys.modules.get("tests.gpu_util")
    rows = getattr(gu, "MARGINS", None) if gu else None
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity margins (max abs error vs the oracle)")
    for case, eo, el, tol in rows:
        tr.write_line(f"{case:<58s} out {eo:.3e}  lse {el:.3e}  tol {tol:.0e}  "
                      f"margin {tol / max(eo, el, 1e-30):.1f}x")
