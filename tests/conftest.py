import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The parity margins the GPU tests measured (worst error / tolerance bound per case),
    printed at the end of the run so that a quiet run's log carries them."""
    sup = sys.modules.get("_support")
    margins = getattr(sup, "MARGINS", None) if sup else None
    if not margins:
        return
    terminalreporter.write_sep("-", "parity margins: worst error / tolerance bound per case (attention: 1e-3 max|o_ref| + 1e-5)")
    for tag, worst in margins:
        terminalreporter.write_line(f"{worst:9.3g}  {tag}")
