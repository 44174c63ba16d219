import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (exhaustive sweeps)")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built on first use if its library is missing)."""
    from oracle import oracle as o
    o._load()
    return o


def pytest_terminal_summary(terminalreporter):
    """GEMM comparisons of the session: how many outputs were checked
    against the oracle and how many passed only through the fp8 MFMA
    accumulation bound (never hidden)."""
    from tests.gpu_util import STATS
    if STATS["comparisons"]:
        terminalreporter.write_line(
            f"GEMM parity: {STATS['comparisons']} comparisons, {STATS['compared']} outputs "
            f"compared; {STATS['with_outside']} comparisons had outputs outside 1e-2|r|+ulp, "
            f"{STATS['outside']} outputs in all, each within the accumulation bound")
