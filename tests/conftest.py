import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(autouse=True)
def _gpu_guard(request):
    """A gpu-marked test never passes silently without a GPU."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        assert torch.cuda.is_available(), "gpu test needs a visible GPU"
    yield


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    _oracle._load()
    return _oracle
