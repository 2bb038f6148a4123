import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    config.addinivalue_line("markers", "fullsize: GPU parity at a bench workload's full size (its errors are "
                            "summarised at the end of the session)")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a visible device; on a CPU-only machine they are skipped
    # rather than silently routed anywhere else.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


_FULL = set()


def pytest_collection_finish(session):
    for item in session.items:
        if "fullsize" in item.keywords:
            _FULL.add(item.nodeid)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Achieved max|err|/rms of the full-size GPU parity cases (raw, and the bf16 compute
    error after each element's own output rounding), one line per compared output."""
    try:
        from tests.gpu_util import RECORDS
    except Exception:  # pragma: no cover
        return
    rows = [r for r in RECORDS if r[0] in _FULL]
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("=", "parity errors at full size (max|err| / rms of the oracle output)")
    for test, qty, raw, comp in rows:
        name = test.split("::", 1)[-1]
        c = "" if comp is None else f"  compute {comp:.3e}"
        tr.write_line(f"PARITY {name} {qty}: raw {raw:.3e}{c}")
