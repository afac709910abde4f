import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes on the GPU box)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its binding, on cuda:0; fails loudly if either
    the GPU or the built library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import second_order_optimizer_amd as kfac
    kfac.load()  # raises if the shared library is absent
    return kfac
