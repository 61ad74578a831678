import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    """Every parity check of the run with its errors against the oracle."""
    from tests import util
    if not util.PARITY_LOG:
        return
    tr = terminalreporter
    tr.section("parity against the fp64 oracle (max normalised error)")
    for what, dtype, eo, el in util.PARITY_LOG:
        tr.write_line(f"{what:<60s} {dtype:>5s}  err_O={eo:.3e} (tol {util.O_TOL[dtype]:.0e})"
                      f"  err_LSE={el:.3e} (tol {util.LSE_TOL[dtype]:.0e})")
