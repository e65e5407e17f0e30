import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case")


def golden(key):
    path = os.path.join(ROOT, "tests", "golden", "page_values.txt")
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, rest = line.split("=", 1)
            if k.strip() == key:
                return float(rest.split("|", 1)[0])
    raise KeyError(key)


@pytest.fixture
def page_value():
    return golden
