import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs a ROCm GPU (MI355X); runs the HIP library through its C ABI")


@pytest.fixture
def gpu():
    """GPU tests fail (not skip) without a GPU: they must never pass silently."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("this test needs a ROCm GPU; run CPU tests with -m 'not gpu'")
    return torch.device("cuda:0")
