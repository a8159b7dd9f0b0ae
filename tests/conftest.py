import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle run")


def pytest_collection_modifyitems(config, items):
    # GPU tests run in file order after the CPU ones; nothing to reorder.
    return


@pytest.fixture(autouse=True)
def _gpu_guard(request):
    """GPU tests need a visible GPU; where one is visible, a missing library still fails loudly."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.skip("no GPU visible")
        print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
