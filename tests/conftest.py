import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (minutes of CPU oracle work)")


def read_golden(name):
    """Non-comment lines of a golden fixture, split into tokens."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
