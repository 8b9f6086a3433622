import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Rows of a whitespace-separated fixture, '#' comments dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture
def golden():
    return read_golden


def pytest_terminal_summary(terminalreporter):
    """Print the parity tally of the GPU checks (tests/parity.py): per compared
    set, the worst error, the relative RMS and the elements beyond the
    per-element bound (admitted by a derived rounding bound, or reported only
    against the oracle with unrounded projections)."""
    try:
        from parity import TALLY
    except ImportError:
        return
    if not TALLY:
        return
    tr = terminalreporter
    tr.section("parity tally")
    tot = {"bound": [0, 0], "derived": [0, 0], "rms": [0, 0]}
    for name, n, beyond, mx, rr, kind in TALLY:
        tot[kind][0] += n
        tot[kind][1] += beyond
        tr.write_line(f"{kind:7s} {name}: n={n} beyond_element_bound={beyond} max_abs={mx:.3e} rel_rms={rr:.3e}")
    for kind, (n, b) in tot.items():
        if n:
            tr.write_line(f"total {kind}: {n} elements, {b} beyond the element bound")
