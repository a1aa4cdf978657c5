import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def ora():
    import oracle
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The session's near-tie tally (printed also under -q)."""
    from tests.gpu_util import TALLY
    n, e = TALLY["compared"], TALLY["excused"]
    if n:
        terminalreporter.write_line(
            f"parity tally: {e} near-tie mismatches excused of {n} tokens and acceptance "
            f"decisions compared ({100.0 * e / n:.4f} %, budget 0.1 %) over "
            f"{len(TALLY['cases'])} cases")
