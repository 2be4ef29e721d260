import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running")


def pytest_terminal_summary(terminalreporter):
    """Repeat the per-workload parity lines that tests/_gpu.py::table gathered, so that they
    appear in quiet runs too."""
    gpu_helpers = sys.modules.get("tests._gpu")
    lines = getattr(gpu_helpers, "TABLE_LINES", None)
    if lines:
        terminalreporter.section("parity table (error against the float64 oracle)")
        for line in lines:
            terminalreporter.write_line(line)


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "closed_form.json")) as f:
        return json.load(f)
