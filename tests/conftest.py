import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def lvq_lib():
    """The built HIP library (GPU tests only); fails loudly when it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_loop_amd import _abi
    return _abi.lib()
