import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture of 'key = value' lines."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            if "," in v:
                out[k] = tuple(float(x) if "." in x else int(x) for x in v.split(","))
            elif "." in v:
                out[k] = float(v)
            else:
                out[k] = int(v)
    return out


@pytest.fixture(scope="session")
def golden_printed():
    return load_golden("smollm2_q8_0_printed.txt")
