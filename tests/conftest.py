import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes tens of seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library through its Python binding; fails loudly without a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected but torch sees no GPU")
    from nvfp4_w4a4_gemm_quantize_amd import binding
    binding.load()
    return binding
