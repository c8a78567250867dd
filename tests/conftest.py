import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is present; returns the loaded library binding."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_17_amd import binding
    return binding.lib()
