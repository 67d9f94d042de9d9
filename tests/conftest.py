import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle run")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    from tests import metrics

    if metrics.LINES:
        terminalreporter.section("parity figures")
        for line in metrics.LINES:
            terminalreporter.write_line(line)
