import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    # The build script is loaded by path: importing the package would first
    # try to load a library that may not exist yet.
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "w4_build", os.path.join(ROOT, "bit_group_quantized_w4_amd", "_build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    if not build.built():
        build.build(verbose=False)


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
