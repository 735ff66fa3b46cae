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
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Print the parity margins the GPU tests recorded (max err / max |oracle|)."""
    try:
        from _gpu_common import MARGINS
    except ImportError:
        return
    if not MARGINS:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity: max |err| / max |oracle| (tolerance)")
    for r in MARGINS:
        tr.write_line(f"{r['case']:<44s} {r['phase']:<18s} {r['max_err_over_max_ref']:.3e}  (tol {r['tol']:.0e})")
