import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built library on a visible GPU; the GPU tests fail loudly without it."""
    import torch
    import attention_forward_online_attn_amd as attn
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    lib = attn.load_library()
    return lib
