import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _has_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """Report the attention output checks: count and the worst max-abs error
    relative to the oracle's RMS and to its largest magnitude."""
    try:
        from tests.parity_util import REPORT
    except Exception:
        return
    if not REPORT:
        return
    tr = terminalreporter
    rel = [(mx / rms if rms else 0.0, mx / big if big else 0.0, mx, what) for what, mx, rms, big in REPORT]
    tr.write_sep("-", f"attention output checks: {len(REPORT)}")
    for r_rms, r_big, mx, what in sorted(rel, reverse=True)[:8]:
        tr.write_line(f"  max-abs {mx:.3e}  /rms {r_rms:.3e}  /max|ref| {r_big:.3e}  {what}")
    worst = max(rel)
    tr.write_line(f"  worst max-abs/rms(oracle) {worst[0]:.3e}; worst max-abs/max|oracle| "
                  f"{max(r[1] for r in rel):.3e}; largest max-abs {max(r[2] for r in rel):.3e}")
