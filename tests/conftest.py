import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library, loaded through the Python binding (GPU tests only)."""
    if not gpu_available():
        pytest.skip("no GPU")
    import fp8_grouped_gemm_ragged_amd as g

    g.load()  # raises if the shared library is missing: no fallback
    return g


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stdout (flushed) before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    yield
