import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def root_dir():
    return ROOT


def pytest_sessionfinish(session, exitstatus):
    """With SDPA14_PARITY_REPORT set, write every output comparison of the
    session (strict maximum, rounding floor, exempt count) as JSON lines."""
    path = os.environ.get("SDPA14_PARITY_REPORT")
    if not path:
        return
    import json

    from tests import _util

    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        for r in _util.REPORT:
            f.write(json.dumps(r) + "\n")
