import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


# Parity summaries of the full-size cases, printed at the end of the run (so that the record of
# a GPU run shows each workload's largest logit difference and near ties, not only pass/fail).
_PARITY = []


@pytest.fixture
def parity_log():
    def log(name, rep):
        _PARITY.append((name, rep.summary().split("\n")[0]))
        print(name, rep.summary())
    return log


def pytest_terminal_summary(terminalreporter):
    if _PARITY:
        terminalreporter.write_sep("-", "oracle parity at full size (teacher-forced)")
        for name, line in _PARITY:
            terminalreporter.write_line(f"{name}: {line}")
