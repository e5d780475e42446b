import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests run in file order; nothing to reorder.  Report the test name
    # before each GPU test so a fault on the box names its case.
    pass


@pytest.fixture(autouse=True)
def _announce(request):
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield
