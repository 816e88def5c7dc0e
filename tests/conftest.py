import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU work")


def to_np(t):
    """bf16/float torch tensor -> float32 numpy (exact for bf16 values)."""
    return t.float().numpy()


@pytest.fixture(scope="session")
def np_of():
    return to_np
