import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # The oracle library is compiled only by its build(); a fresh checkout
    # gets it here, before any test has touched a GPU (a process that has
    # initialised one must not start a compiler).
    import oracle
    if not os.path.exists(oracle._LIB):
        oracle.build()


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
