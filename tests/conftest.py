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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (test infrastructure); built with gcc if nothing is built."""
    from oracle import oracle as oracle_mod
    if not os.path.exists(oracle_mod.DEFAULT_LIB):
        from oracle import build as oracle_build
        oracle_build.build()
    return oracle_mod.default()
