import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload (seconds of CPU oracle time)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib_path():
    """Path of the built C-ABI library; builds it once if it is missing."""
    from fp8_block_scaled_04_amd import build as b
    path = b.library_path()
    if not os.path.exists(path):
        b.build_library()
    return path
