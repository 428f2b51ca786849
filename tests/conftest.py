import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library bound through its C ABI; GPU tests fail (never fall back) without it."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU")
    from token_scoring_eviction_amd import kvc
    kvc.load()
    return kvc


@pytest.fixture
def kvc_option(gpu_lib):
    """Sets libkvc's process-wide options (kvc_set_option) for one test; every option
    goes back to its default afterwards."""
    yield gpu_lib.kvc_set_option
    for name, value in gpu_lib.OPTION_DEFAULTS.items():
        gpu_lib.kvc_set_option(name, value)
