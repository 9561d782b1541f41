import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (seconds to a minute)")


def pytest_collection_modifyitems(config, items):
    # GPU tests print what they run first, so a box that dies mid-run still
    # names the case in the captured output.
    pass


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle as o
    o.lib()
    return o
