import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.default_oracle()


@pytest.fixture(scope="session")
def mhla_lib():
    """libmhla.so, built first only if it is missing (the build needs no GPU)."""
    import token_level_head_amd as mh
    from token_level_head_amd import build

    if not os.path.exists(mh.LIB_PATH):
        build.build()
    return mh.load_library()
