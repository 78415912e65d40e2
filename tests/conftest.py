import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a tests/golden fixture: 'key v1 v2 ...' lines, '#' comments, ';' separates rows."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            if ";" in rest:
                out[key] = [[float(t) for t in part.split()] for part in rest.split(";")]
            else:
                vals = [float(t) for t in rest.split()]
                out[key] = vals[0] if len(vals) == 1 else vals
    return out


@pytest.fixture
def golden():
    return read_golden
