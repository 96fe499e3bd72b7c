import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running GPU test at full workload size")


@pytest.fixture(scope="session")
def kvq_lib():
    """The HIP library through its binding; builds it in-tree if nothing is built."""
    from quantized_kv_cache_append_amd import binding
    if not binding.library_path_exists():
        import __graft_entry__
        __graft_entry__.build()
    return binding.load()
