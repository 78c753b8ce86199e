import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads; minutes of oracle time on the host")


def pytest_collection_modifyitems(config, items):
    # A GPU test on a host without a GPU is skipped, not failed, so `-m "not gpu"` and a bare
    # `pytest` both work in a CPU-only container.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per named workload with the errors its parity test measured (max abs error and
    relative RMS of O over the whole output, largest LSE error), so a quiet run still shows them."""
    try:
        import parity
    except ImportError:  # pragma: no cover
        return
    if not parity.SUMMARY:
        return
    tr = terminalreporter
    tr.section("parity against the fp64 oracle (whole outputs)")
    for name, st in parity.SUMMARY:
        parts = [f"{k} {v:.3g}" if isinstance(v, float) else f"{k} {v}" for k, v in st.items()]
        tr.write_line(f"{name}: " + ", ".join(parts))
