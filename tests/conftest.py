import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_host_libs():
    """Build the host-only libraries if they are missing (gcc, seconds)."""
    from sparse_mla_attention_indexer_amd import _build
    import oracle

    if not os.path.exists(_build.WORKLOAD_LIB):
        _build.build_workload()
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()


_ensure_host_libs()


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def hip_lib():
    """The HIP library; GPU tests need it built in-tree and fail loudly if it is not."""
    from sparse_mla_attention_indexer_amd import _lib

    return _lib.lib()
