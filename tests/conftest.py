import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload (seconds of oracle time)")


@pytest.fixture(scope="session")
def nrm_lib():
    """The HIP library through its Python binding; GPU tests only."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import transformer_row_wise_amd as nrm

    nrm.load()  # raises if the HIP library is missing: never a silent fallback
    return nrm
