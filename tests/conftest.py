import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP device (MI355X); runs the HIP library")
    config.addinivalue_line("markers", "slow: large CPU work; still part of the default suite")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library on cuda:0. A GPU test without a device fails loudly."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test needs a HIP device; run it on the MI355X (tests marked gpu)")
    import paged_kv_cache_49_amd as pa
    pa.lib()  # raises if the shared library is missing
    return pa
