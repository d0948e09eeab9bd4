import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _default_dtype_unchanged():
    """Every test must leave torch's default dtype at float32: a leaked float64 default
    silently changes the dtype of tensors other tests build without an explicit one."""
    yield
    import torch
    assert torch.get_default_dtype() == torch.float32, (
        "test left the torch default dtype at %s" % torch.get_default_dtype())
