import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library, loaded through the binding; fails loudly when absent."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import speculative_decode_verify_mla_amd as mv

    mv.load_library()
    return mv
