import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case, minutes of CPU oracle time")


@pytest.fixture(scope="session")
def lib():
    """The loaded C-ABI library; on a machine with the GPU a missing build is an error, not a skip."""
    from exact_tiled_attention_25_amd import binding
    return binding.load()
