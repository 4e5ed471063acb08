import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip-free guard: a gpu-marked test on a machine without a GPU is an error,
    except when the whole gpu tier is deselected (``-m "not gpu"``)."""
    if not _gpu_available():
        pytest.fail("gpu-marked test started but torch sees no GPU")
    import torch
    return torch.device("cuda", 0)


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library through its Python binding (loads without a GPU)."""
    import structured_sparse_gemm_w24_amd as ssg
    return ssg
