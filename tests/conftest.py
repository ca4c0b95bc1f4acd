import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)

import _parity_log  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Observed parity figures of the GPU tests, printed last so that the
    tail of the run carries them, and written as JSON."""
    lines = _parity_log.summary_lines()
    if not lines:
        return
    path = _parity_log.write_json()
    for line in lines:
        terminalreporter.write_line(line)
    if path:
        terminalreporter.write_line(f"  all figures: {path}")
