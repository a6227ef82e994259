import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle work of tens of seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; only for tests marked gpu."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import exact_tiled_attention_32_amd as fa
    fa.load()  # raises if the HIP library is missing
    return fa
