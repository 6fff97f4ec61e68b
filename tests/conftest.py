import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=not os.path.exists(os.path.join(ROOT, "oracle", "libmxref.so")))
    return oracle


GOLDEN = os.path.join(ROOT, "tests", "golden")


def golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows
