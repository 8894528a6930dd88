import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) where there is no GPU, so that a plain
    # `pytest` on a CPU host still runs the oracle and host-side tests.
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


def pytest_terminal_summary(terminalreporter):
    # the per-output parity lines collected by parity_util (GEMM1 intermediate
    # flips and the share of the tolerance their allowance took)
    try:
        from parity_util import SUMMARY
    except Exception:  # pragma: no cover
        return
    if SUMMARY:
        terminalreporter.section("parity summary")
        for line in SUMMARY:
            terminalreporter.write_line(line)
