import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU statistics test")


def pytest_collection_modifyitems(config, items):
    # GPU tests go last so a CPU failure is reported before any GPU work starts
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per GPU comparison: matches and excused draws (counted, never
    hidden), so the round's log shows how often the 1e-6 window was used."""
    try:
        from parity_util import SESSION_COUNTS
    except ImportError:
        return
    if not SESSION_COUNTS:
        return
    tr = terminalreporter
    tr.section("GPU-vs-oracle comparison counts")
    tot = {}
    for label, c in SESSION_COUNTS:
        tr.write_line(f"{label}: {c}")
        for key, v in c.items():
            tot[key] = tot.get(key, 0) + v
    tr.write_line(f"TOTAL: {tot}")
