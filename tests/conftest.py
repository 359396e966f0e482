import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture: 'key = v v ; v v' lines, '#' comments."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (x.strip() for x in line.split("=", 1))
            rows = [[float(t) for t in r.split()] for r in val.split(";")]
            out[key] = rows[0][0] if len(rows) == 1 and len(rows[0]) == 1 else rows
    return out


@pytest.fixture
def golden():
    return read_golden
