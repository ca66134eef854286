import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lad():
    """The GPU library's Python binding.  Loading fails loudly when the HIP
    extension is missing: there is no CPU fallback."""
    if not gpu_available():
        pytest.skip("no GPU")
    from sparse_autodiff_mesh_amd import binding
    return binding
