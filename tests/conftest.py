import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Parse a ``key = value`` fixture (``#`` comments). Values with spaces become lists."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line or "=" not in line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            parts = v.split()
            conv = []
            for p in parts:
                try:
                    conv.append(int(p))
                except ValueError:
                    conv.append(float(p))
            out[k] = conv if len(conv) > 1 else conv[0]
    return out


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(v) for v in line.split()])
    return rows


@pytest.fixture(scope="session")
def golden():
    return read_golden


@pytest.fixture(scope="session")
def golden_table():
    return read_table
