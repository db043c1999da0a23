import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


_SUMMARY = []


def record_summary(line: str) -> None:
    """A line for the end-of-run summary (parity counts of the full-size cases)."""
    _SUMMARY.append(line)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if _SUMMARY:
        terminalreporter.section("parity summary")
        for line in _SUMMARY:
            terminalreporter.write_line(line)


@pytest.fixture(autouse=True)
def _library_output_guards(request):
    """After every GPU test: no library call wrote past the buffers the test
    handed it (guard regions around them, tests/parity.py)."""
    yield
    if request.node.get_closest_marker("gpu") is not None:
        from tests.parity import check_guards
        check_guards()
