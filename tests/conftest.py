import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, on a machine with a GPU.  Fails (never skips) when no
    GPU or no built library is present: a gpu-marked test must not pass on a
    fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test run without a visible GPU")
    import linear_attention_phi_amd as la
    la.load()  # raises if the HIP library is missing
    return la
