import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_mod():
    from oracle import oracle as o
    o.build(force=False)
    return o


@pytest.fixture(scope="session")
def built_lib():
    """libspt.so as built in-tree; built here only when it is missing."""
    from software_pipelined_tiling_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    return b.LIB


@pytest.fixture(scope="session")
def poison_lib():
    """libspt_poison.so (the race-detection build) as built in-tree; built here only when it is missing."""
    from software_pipelined_tiling_amd import build as b
    if not os.path.exists(b.POISON_LIB):
        b.build_poison()
    return b.POISON_LIB
