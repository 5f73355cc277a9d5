import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def lib():
    """The loaded C-ABI library (skips the test when it has not been built)."""
    from paged_kv_cache_222_amd import _binding
    if not os.path.exists(_binding.library_path()):
        pytest.skip("libpa.so not built")
    return _binding.load()
