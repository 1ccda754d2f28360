import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture: 'key value [tolerance] citation...' per line."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip() if line.lstrip().startswith("#") else line.strip()
            if not line:
                continue
            parts = line.split()
            key, val = parts[0], parts[1]
            v = int(val, 16) if val.lower().startswith("0x") else float(val)
            tol = None
            if len(parts) > 2:
                try:
                    tol = float(parts[2])
                except ValueError:
                    tol = None
            out[key] = (v, tol)
    return out


@pytest.fixture
def golden():
    return read_golden
