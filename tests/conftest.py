import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu():
    """Skip-free GPU fixture: a gpu-marked test needs a GPU and the built
    library; a missing GPU is an error, not a skip."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test needs a GPU")
    from quantize_grouped_gemm_amd import mx
    mx.lib()  # raises if libmxfp8.so is missing or fails to load
    return torch.device("cuda:0")
