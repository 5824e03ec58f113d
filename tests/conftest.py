import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture: 'key: numbers' lines, '#' comments."""
    import numpy as np
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, vals = line.split(":", 1)
            out[key.strip()] = np.array([float(x) for x in vals.split()], dtype=np.float64)
    return out


@pytest.fixture(scope="session")
def golden():
    return load_golden
