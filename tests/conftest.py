import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests of the HIP path")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU or GPU work)")


def read_golden(name: str) -> dict:
    """Parse a tests/golden fixture: '#' comments, then 'key: v1 v2 ...' lines."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.split()
    return out


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle
