import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity cases")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library on cuda:0; fails loudly when the extension is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine with no GPU")
    from exact_attention_fa_amd import _lib
    _lib.load()
    return _lib
