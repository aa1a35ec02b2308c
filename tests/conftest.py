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
    if not _gpu_available():
        pytest.skip("no GPU visible")
    import torch
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def lib():
    """The HIP library binding; GPU tests fail (not skip) when it is not built."""
    import grouped_gemm_qgemm_amd as q
    q.load()
    return q
