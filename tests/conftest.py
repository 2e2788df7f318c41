import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU oracle work")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP binding, loaded once; fails loudly when the library or GPU is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch sees no GPU")
    import linear_memory_relation_amd as lmr
    lmr.load()      # raises if the built library is missing
    return lmr


# Parity figures that the GPU tests print (loss_rel, max-rel errors) are
# repeated in a section of the terminal summary, so that a quiet run's log
# still carries them.
_PARITY_KEYS = ("loss_rel", "maxrel", "max-rel", "lse_err", "kl_err")
_parity_lines = []


def pytest_runtest_logreport(report):
    if report.when == "call" and report.passed and report.capstdout:
        for line in report.capstdout.splitlines():
            if any(k in line for k in _PARITY_KEYS):
                _parity_lines.append(f"{report.nodeid.split('::')[-1]}: {line.strip()}")


def pytest_terminal_summary(terminalreporter):
    if _parity_lines:
        terminalreporter.section("parity figures printed by the passing tests")
        for line in _parity_lines:
            terminalreporter.write_line(line)
