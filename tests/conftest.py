import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU-side case (still minutes at most)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Near-tie counts and the worst used fraction of each tolerance
    (elementwise err/limit, then normwise err/rtol) of the GPU parity tests."""
    try:
        from _helpers import REPORT
    except ImportError:
        return
    if REPORT:
        terminalreporter.write_line("parity report (used tolerance: elementwise / normwise):")
        for line in REPORT:
            terminalreporter.write_line("  " + line)
