import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a ``name = value | citation`` fixture under tests/golden/."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0] if line.lstrip().startswith("#") else line
            if "=" not in line:
                continue
            key, rest = line.split("=", 1)
            out[key.strip()] = float(rest.split("|", 1)[0].strip())
    return out


@pytest.fixture(scope="session")
def page_constants():
    return read_golden("page_constants.txt")


@pytest.fixture(scope="session")
def closed_forms():
    return read_golden("closed_forms.txt")
