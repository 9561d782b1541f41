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


@pytest.fixture(scope="session")
def gq_lib_path():
    """Path of libgq.so; built here (hipcc cross-compiles for gfx950 without a
    GPU) if it is missing."""
    path = os.path.join(ROOT, "block_quantized_weight_q4_amd", "libgq.so")
    if not os.path.exists(path):
        from block_quantized_weight_q4_amd import build
        build.build()
    return path
