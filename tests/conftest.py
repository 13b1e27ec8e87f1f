import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU (MI355X)")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def dsa():
    """The HIP binding; fails (not skips) when the library is missing on a machine with a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_amd as m
    m.load_library()
    return m
