import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def ref():
    """The CPU oracle (built with gcc if nothing is built yet)."""
    from oracle import build, oracle
    if not os.path.exists(oracle.LIB_PATH):
        build.build()
    return oracle


def read_golden(name):
    path = os.path.join(ROOT, "tests", "golden", name)
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [float(x) for x in rest]
    return vals
