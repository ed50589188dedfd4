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
def gpu_lib():
    """The HIP library bound through ctypes, on a GPU machine only."""
    import torch  # noqa: F401  (loads the HIP runtime the library links against)
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from vision_transformer_amd import vitenc
    return vitenc.lib()
