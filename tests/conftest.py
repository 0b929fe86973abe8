import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_collection_modifyitems(config, items):
    # GPU tests refuse to run without a device rather than silently passing.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    try:
        from margins import RECORDS
    except ImportError:  # pragma: no cover
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.section("parity margins (error / bound)")
    for case, what, err, bound in RECORDS:
        tr.write_line(f"{case:60s} {what:>14s} {err:10.3e} <= {bound:8.1e}  ({err / bound:6.3f} of the bound)")
