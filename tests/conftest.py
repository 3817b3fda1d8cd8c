import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded C-ABI library; only for tests marked gpu."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from depth_recurrent_layer_amd import dreamer
    return dreamer
