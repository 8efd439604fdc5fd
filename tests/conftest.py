import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an AMD Instinct GPU (gfx950) and the HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def read_golden(name):
    path = os.path.join(ROOT, "tests", "golden", name)
    with open(path) as f:
        return [ln.rstrip("\n") for ln in f if ln.strip() and not ln.startswith("#")]
