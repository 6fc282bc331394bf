import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(autouse=True)
def _gpu_required(request):
    """A selected `gpu` test fails (it is not skipped) when no GPU is visible:
    a GPU suite run on a machine without one must not report success."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch

        if not torch.cuda.is_available():
            pytest.fail("gpu test selected but no GPU is visible", pytrace=False)
    yield
