import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; fails rather than skips without one")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    from oracle import build
    build.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The binding, on a GPU that must be there (a missing GPU is a failure)."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import quantized_weight_prefill_gguf_amd as pf
    pf.load()
    return pf
