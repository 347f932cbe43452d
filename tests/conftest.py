import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libfa.so")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def fa_lib():
    """The built HIP library, loaded (built first only if nothing is built)."""
    from exact_io_aware_fa_amd import binding
    if not os.path.exists(binding.library_path()):
        from exact_io_aware_fa_amd import build as fa_build
        fa_build.build()
    return binding.load_library()
