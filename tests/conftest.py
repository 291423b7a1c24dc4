import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, on a machine with a GPU. Fails (does not skip) when the
    library is missing: a GPU run must exercise the native path."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import block_scaled_fp8_fp8blk_amd as fb
    fb.load()  # raises if the shared library is absent
    return fb
