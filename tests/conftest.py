import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import parity_bars  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.hookimpl(hookwrapper=True)
def pytest_runtest_call(item):
    parity_bars.CURRENT[0] = item.nodeid.split("::", 1)[-1]
    yield
    parity_bars.CURRENT[0] = ""


def pytest_terminal_summary(terminalreporter):
    lines = parity_bars.summary_lines()
    if not lines:
        return
    terminalreporter.section("parity margins")
    for ln in lines:
        terminalreporter.write_line(ln)
    path = os.environ.get("SAS_MARGINS_JSON")
    if path:
        with open(path, "w") as f:
            json.dump(parity_bars.RECORD, f, indent=1, sort_keys=True)


@pytest.fixture(scope="session")
def repo_root():
    return ROOT
