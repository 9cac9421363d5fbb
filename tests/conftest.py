import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session")
def cuda():
    """The GPU and the built HIP library; GPU tests never fall back to the CPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from self_speculative_decoding_w4a16_amd import _lib
    _lib.lib()  # raises if libsubspec.so is missing
    return torch.device("cuda:0")
