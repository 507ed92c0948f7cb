import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads")


def pytest_collection_modifyitems(config, items):
    # GPU-less hosts: GPU tests still get collected; they skip themselves in the fixture.
    pass


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; skips when no GPU is visible."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import mla_paged_kv_metadata_amd as mla

    mla.load_library()   # raises if the HIP library is missing: no silent fallback
    return mla
