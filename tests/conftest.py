import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Lines of a golden fixture with comments and blank lines removed."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded for GPU tests; fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from weight_only_quantized_quantize_amd import woq
    woq.require_gpu()
    return woq
