import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def rr_lib():
    """The HIP library through its Python binding; skips when no GPU is present."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_block_sparse_rr_amd as rr

    rr.load()
    return rr


def pytest_terminal_summary(terminalreporter):
    from tests import report

    if report.LINES:
        terminalreporter.write_sep("-", "workload parity: block-list rows by class, attention rows compared")
        for line in report.LINES:
            terminalreporter.write_line(line)
