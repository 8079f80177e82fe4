import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_collection_modifyitems(config, items):
    """tests/test_abi.py feeds the library fake device addresses.  Where a GPU can be
    reached, those tests run only inside test_in_child_without_gpu's child process (no
    visible GPU); elsewhere they run directly and the child runner is dropped."""
    gpu_reachable = os.path.exists("/dev/kfd")
    child = os.environ.get("SMOE_ABI_CHILD") == "1"
    keep, drop = [], []
    for it in items:
        in_abi = os.path.basename(str(it.fspath)) == "test_abi.py"
        runner = in_abi and it.name == "test_in_child_without_gpu"
        if in_abi and ((gpu_reachable and not child) != runner):
            drop.append(it)
        else:
            keep.append(it)
    if drop:
        config.hook.pytest_deselected(items=drop)
        items[:] = keep
