import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, where no GPU is visible (this keeps the
    # CPU suite green); on a GPU machine they run against the built HIP library.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    # one line per full-size comparison (max / mean |dO|, max |dLSE|), so the
    # errors of every workload show in the run's summary, not only on failure
    lines = []
    for key in ("passed", "failed"):
        for rep in terminalreporter.stats.get(key, []):
            if getattr(rep, "when", "call") != "call":
                continue
            for name, value in getattr(rep, "user_properties", []):
                if name == "parity":
                    lines.append(("PASS " if key == "passed" else "FAIL ") + str(value))
    if lines:
        terminalreporter.write_sep("-", "parity against the fp64 oracle")
        for line in lines:
            terminalreporter.write_line(line)
