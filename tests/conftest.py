import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def golden(name):
    """Parse tests/golden/<name>: 'key = v1 v2 ...' lines, '#' comments."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            vals = [float(v) if "." in v else int(v) for v in val.split()]
            out[key] = vals[0] if len(vals) == 1 else vals
    return out


@pytest.fixture
def gold():
    return golden
