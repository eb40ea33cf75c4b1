import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu():
    """The loaded HIP library; fails (never skips) when no GPU is visible or the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu test run without a visible GPU")
    import decode_attention_paged_gqa_amd as da

    da.load()  # raises if the built library is absent
    return da
