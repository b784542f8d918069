import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def read_golden(name):
    """Rows of a tests/golden text fixture, comments and blank lines removed."""
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("|")[0].strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows
