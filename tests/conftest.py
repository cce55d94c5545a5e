import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    host_lib = os.environ.get("PA_TEST_HOST_LIB")
    if host_lib:
        _use_host_library(host_lib)


def _use_host_library(path):
    """Point the binding's host calls at another build of the block manager
    (the sanitized host-only library of tests/test_host_sanitized.py).  Device
    entry points are absent from it, so a test that reaches one fails."""
    import ctypes

    import paged_kv_cache_394_amd as pa
    lib = ctypes.CDLL(path)
    for name, (res, args) in pa._SIGNATURES.items():
        if hasattr(lib, name):
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
    pa.lib = lib


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
