import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")
    config.addinivalue_line("markers", "slow: larger CPU oracle cases")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding with a visible GPU; tests that take it are marked ``gpu``."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import post_weight_quantization_amd as pwq
    pwq.require_native()
    return pwq
