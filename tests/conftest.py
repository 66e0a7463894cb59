import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def qmv_gpu():
    """The HIP library bound to cuda:0; the test fails (not skips) if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from ternary_matvec_amd import qmv
    lib = qmv.load()
    return lib
