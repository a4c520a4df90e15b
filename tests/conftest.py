import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded C-ABI library with a visible GPU; GPU tests fail loudly if
    either is missing (no CPU fallback exists)."""
    import torch
    import rotation_bit_ptq_amd as rbp
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return rbp
