import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Build libhsa.so in-tree when it is not there yet (hipcc cross-compiles without a GPU)."""
    from token_sparse_attention_compact_amd import hsa
    if not os.path.exists(hsa.lib_path()):
        from token_sparse_attention_compact_amd import build
        build.build()
    yield
