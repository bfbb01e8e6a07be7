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


@pytest.fixture(params=["auto", "big"])
def gemm_tile(request, monkeypatch):
    """Run a GPU test with the library's own tile choice and with the large
    tiles forced: 256 x 256 for bf16 products (DMUON_GEMM_TILE), 128 x 128
    for fp32 ones (DMUON_GEMM_TILE_F32)."""
    if request.param == "auto":
        monkeypatch.delenv("DMUON_GEMM_TILE", raising=False)
        monkeypatch.delenv("DMUON_GEMM_TILE_F32", raising=False)
    else:
        monkeypatch.setenv("DMUON_GEMM_TILE", "256")
        monkeypatch.setenv("DMUON_GEMM_TILE_F32", "128")
    return request.param
