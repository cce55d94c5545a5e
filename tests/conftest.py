import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests print the case they run before touching the device, so a run
    # that ends the process early still names its last case.
    pass


@pytest.fixture(autouse=True)
def _name_the_case(request):
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[case] {request.node.nodeid}", flush=True)
    yield


def load_golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)
