import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture: ``key: values`` lines, ``#`` comments,
    ``case NAME`` lines start a new section (keys are then ``NAME.key``).
    Values: whitespace-separated numbers; ``|`` separates rows."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    prefix = ""
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case "):
                prefix = line.split()[1] + "."
                continue
            key, _, val = line.partition(":")
            rows = [r.split() for r in val.split("|")]
            out[prefix + key.strip()] = rows if len(rows) > 1 else rows[0]
    return out


@pytest.fixture(scope="session")
def golden():
    return read_golden
