import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running sweep")


@pytest.fixture(scope="session")
def lib():
    """The Python binding over the C-ABI library (GPU tests only)."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import invariant_bi_mm_amd as bi
    return bi
