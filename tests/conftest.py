import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


def pytest_terminal_summary(terminalreporter):
    """Error maxima of the parity comparisons: each full-size workload's, and the worst ratio overall."""
    try:
        from tests.util import ERRORS
    except ImportError:  # pragma: no cover
        return
    if not ERRORS:
        return
    tr = terminalreporter
    tr.section("parity error maxima (max-relative per (batch, head) slice)")
    for test, what, err, tol in ERRORS:
        if "full_size" in test or "workload" in test:
            tr.write_line(f"{test} [{what}]: {err:.3e} (tol {tol:.0e})")
    test, what, err, tol = max(ERRORS, key=lambda e: e[2] / e[3] if e[3] > 0 else 0.0)
    tr.write_line(f"{len(ERRORS)} comparisons; largest error / tolerance {err / tol:.3f}: {test} [{what}] "
                  f"{err:.3e} (tol {tol:.0e})")
