import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test, run when FP_SLOW_TESTS=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("FP_SLOW_TESTS") == "1":
        return
    skip = pytest.mark.skip(reason="slow; set FP_SLOW_TESTS=1")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)


def load_golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(autouse=True)
def _skip_gpu_without_device(request):
    if "gpu" in request.keywords and not _gpu_available():
        pytest.skip("no GPU in this environment")


@pytest.fixture(scope="session")
def fp():
    """The HIP library's binding; raises if libflatparam.so is not built."""
    import __graft_entry__
    __graft_entry__._ensure_built()
    import sharded_flatparameter_pack_amd as fp
    fp.lib()
    return fp
