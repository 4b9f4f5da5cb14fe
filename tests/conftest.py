import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library on cuda:0; fails loudly if it is missing."""
    import torch
    from token_level_sparse_pass_amd import hs2
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    hs2.load()          # raises if libhs2.so was not built
    return hs2
