import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle


def pytest_terminal_summary(terminalreporter):
    bars = sys.modules.get("bars")
    if bars is not None and bars.REPORT:
        terminalreporter.section("logits accuracy (|gpu - exact| against the bars in tests/bars.py)")
        for line in bars.REPORT:
            terminalreporter.write_line(line)
