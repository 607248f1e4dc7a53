import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip-free GPU guard: a gpu-marked test on a machine without a GPU is an error."""
    if not _gpu_available():
        pytest.fail("this test needs a GPU (run it with -m gpu on an MI355X)")
    import torch

    return torch.device("cuda:0")
