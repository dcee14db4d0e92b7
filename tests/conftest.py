import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _gpu_available() -> bool:
    try:
        import torch
    except Exception:
        return False
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def gpu():
    """Skips nothing: a gpu-marked test run without a GPU is an error, not a skip."""
    if not _gpu_available():
        pytest.fail("gpu test selected but no GPU is visible")
    import torch

    return torch.device("cuda:0")
