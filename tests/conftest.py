import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libarl2")
    config.addinivalue_line("markers", "slow: long-running parity case")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


def pytest_terminal_summary(terminalreporter):
    """Host time the float64 oracle took in the parity tests, per workload."""
    pu = sys.modules.get("parity_utils")
    if pu is None or not pu.ORACLE_SECONDS:
        return
    terminalreporter.write_sep("-", f"oracle wall time in the parity tests ({pu.oracle_threads()})")
    for name, sec in sorted(pu.ORACLE_SECONDS.items()):
        terminalreporter.write_line(f"oracle {name}: {sec * 1e3:.1f} ms")
