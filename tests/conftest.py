import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on cuda:0; a missing GPU or library is an error, never a fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU: run with -m 'not gpu' here")
    from mixture_experts_routed_router_amd import _lib
    _lib.load()  # raises if the built library is missing
    return _lib
