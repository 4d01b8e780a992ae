import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is visible; fail loudly if the HIP library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import combine_ep_dispatch_amd as ep  # raises if libep.so is absent

    return ep
