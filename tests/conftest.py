import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library's Python binding, on a machine with a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_verify_attention_amd as tva
    tva.load()          # raises if the built library is missing
    return tva
