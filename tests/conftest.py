import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library through its Python binding (GPU tests only)."""
    if not gpu_available():
        pytest.skip("no GPU")
    from roofline_attention_amd import binding
    return binding
