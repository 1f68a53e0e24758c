"""Shared pytest set-up: the ``gpu`` marker and import paths.

Tests marked ``gpu`` need an AMD Instinct GPU (gfx950) and the built HIP
library; everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case (oracle at full size)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def _ensure_library():
    """Build libpdllm.so in-tree if it is missing (hipcc cross-compiles for
    gfx950 without a GPU), so the boundary tests always have it to load."""
    lib = os.path.join(ROOT, "diffusion_long_context_amd", "libpdllm.so")
    if not os.path.exists(lib):
        from diffusion_long_context_amd.build import build
        build()


_ensure_library()
