import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


def pytest_terminal_summary(terminalreporter):
    """Counted ties of the acceptance parity checks: decisions within 1e-6 of
    their threshold, where the GPU and the oracle may differ."""
    try:
        import parity
    except ImportError:
        return
    t = parity.TOTALS
    if t["sequences"]:
        terminalreporter.write_line(f"acceptance parity: {t['sequences']} sequences compared with the oracle, "
                                    f"{t['ties']} counted ties")
    if t.get("tree_sequences"):
        terminalreporter.write_line(f"state-tree parity: {t['tree_sequences']} sequences compared with the oracle, "
                                    f"{t['tree_ties']} counted ties")
