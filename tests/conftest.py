import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are collected everywhere; run them with -m gpu on a machine with an MI355X
    # and deselect them with -m "not gpu" elsewhere.
    pass


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
