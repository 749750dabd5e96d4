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
    """The parity figures the full-size tests measured (max|err|/rms per
    workload), shown whatever the capture mode."""
    mod = sys.modules.get("tests.parity")
    if mod is None or not mod.REPORTED:
        return
    terminalreporter.write_sep("-", "parity against the float64 oracle")
    for line in mod.REPORTED:
        terminalreporter.write_line(line)
