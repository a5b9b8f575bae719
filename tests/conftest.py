import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    from bit_group_quantized_w4_amd import _build

    if not _build.built():
        _build.build(verbose=False)


@pytest.fixture(scope="session")
def w4():
    """The Python binding of libw4.so (built in-tree first if nothing is built)."""
    _ensure_built()
    import bit_group_quantized_w4_amd as mod

    return mod


@pytest.fixture(scope="session")
def gpu(w4):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()
    return torch.device("cuda:0")
