import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libgemm")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of GPU time")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def switches():
    """Set libgemm's kernel-choice overrides for one test (binding.TEST_*
    flags, or'ed); they are cleared again when the test ends."""
    from dense_gemm_optimisation_amd import binding
    state = {"flags": 0}

    def set_(*flags):
        f = 0
        for x in flags:
            f |= x
        state["flags"] = f
        binding.test_switches(f)
    set_.clear = lambda: set_()
    set_.add = lambda flag: set_(state["flags"] | flag)
    set_.drop = lambda flag: set_(state["flags"] & ~flag)
    binding.test_switches(0)
    yield set_
    binding.test_switches(0)

