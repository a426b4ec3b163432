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
    """The HIP library binding; skips cleanly only when no GPU is visible."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from dequant_gemm_trellis_amd import trellis

    return trellis
