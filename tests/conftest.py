import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: CPU test taking more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on a real GPU; fails (never falls back) when absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    from draft_verify_sampling_spec_amd import binding
    return binding.load()


def pytest_sessionstart(session):
    """Build the HIP library once if this checkout has none yet."""
    from draft_verify_sampling_spec_amd import build
    if not os.path.exists(build.LIB_PATH):
        build.build_library(verbose=False)
