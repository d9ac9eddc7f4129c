import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    """Print what the GPU parity tests recorded: the full-size every-row
    errors, and for the cases checked against the output-rounding bound how
    many elements went past the flat tolerance (with the floor there)."""
    try:
        from parity_common import FLAT_EXCESS, FULL_SIZE
    except ImportError:
        return
    tr = terminalreporter
    if FULL_SIZE:
        tr.write_sep("-", "full-size workloads, every row against the fp64 oracle")
        for name, rows, err_o, err_l, tol in FULL_SIZE:
            tr.write_line(f"{name}: {rows} rows, max|dO| = {err_o:.4e} (tol {tol:g}), "
                          f"max|dLSE| = {err_l:.4e} (tol 1e-3)")
    if FLAT_EXCESS:
        cases = len(FLAT_EXCESS)
        over = [r for r in FLAT_EXCESS if r[1] > 0]
        tr.write_sep("-", "output-rounding bound: elements past the flat tolerance")
        tr.write_line(f"{cases} cases checked with the rounding bound; {len(over)} have "
                      f"elements past the flat tolerance")
        for name, n, size, err, ref, floor in over:
            tr.write_line(f"  {name}: {n}/{size} elements, worst |dO| = {err:.4e} at "
                          f"|O| = {abs(ref):.3f}, output-rounding floor {floor:.4e}")
