import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build the oracle and the HIP library only if nothing is built yet."""
    import oracle
    if not os.path.exists(oracle.LIB):
        oracle.build()
    from ar_rmsnorm_amd import build as arbuild
    if not os.path.exists(arbuild.LIB):
        arbuild.build()


_ensure_built()


@pytest.fixture(scope="session")
def gpu():
    """The torch device for GPU tests; fails loudly without a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    return torch.device("cuda:0")
