import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes tens of seconds or more (full-size oracle comparisons)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; only for tests marked gpu."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import block_scaled_fp4_sigmoid_amd as bsm

    bsm.load()  # raises if the built library is missing
    return bsm
