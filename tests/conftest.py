import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library through its Python binding (GPU tests only)."""
    if not gpu_available():
        pytest.skip("no GPU")
    import matrix_optimizer_step_owned_amd as dm
    return dm


@pytest.fixture(params=["auto", "256"])
def gemm_tile(request, monkeypatch):
    """Run a GPU test with the library's own tile choice and with the
    256 x 256 bf16 tiles forced (DMUON_GEMM_TILE)."""
    if request.param == "auto":
        monkeypatch.delenv("DMUON_GEMM_TILE", raising=False)
    else:
        monkeypatch.setenv("DMUON_GEMM_TILE", request.param)
    return request.param
