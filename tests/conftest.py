import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests print their case before running, so a crash names it.
    pass


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def gen():
    import gen as g

    g._load()
    return g
