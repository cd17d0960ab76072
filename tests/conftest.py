import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_collection_modifyitems(config, items):
    have_gpu = False
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """The tightest parity margins of the run (error / tolerance), so a quiet run still
    shows how close each bound came."""
    try:
        from gpu_util import MARGINS
    except Exception:
        return
    if not MARGINS:
        return
    worst = {}
    for test, what, err, tol in MARGINS:
        r = err / tol if tol > 0 else (0.0 if err == 0 else float("inf"))
        key = (test, what)
        if key not in worst or r > worst[key][0]:
            worst[key] = (r, err, tol)
    rows = sorted(worst.items(), key=lambda kv: -kv[1][0])
    terminalreporter.write_line(f"parity margins: {len(rows)} bounds checked; tightest (err / tol):")
    for (test, what), (r, err, tol) in rows[:12]:
        terminalreporter.write_line(f"  {r:6.3f}  err {err:.3e} tol {tol:.3e}  {what}  [{test}]")
