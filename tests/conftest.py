import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library on cuda:0.  GPU tests fail, never skip, without a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import paged_kv_cache_240_amd as pa
    pa.load()  # raises if libpa.so is missing: there is no fallback
    return pa


def pytest_runtest_logstart(nodeid, location):
    """Name each test before it runs (flushed), so a GPU fault names its case."""
    sys.stderr.write(f"\n>>> {nodeid}\n")
    sys.stderr.flush()
