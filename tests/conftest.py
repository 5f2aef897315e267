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
    if not (os.path.exists(build.LIB_PATH) and os.path.exists(build.TEST_LIB_PATH)):
        build.build_library(verbose=False)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line with the session's near-tie counts of the sampled parity
    checks (requests whose first diverging decision of the oracle lay within
    the 1e-6 band and were excused), and a JSON record when NEAR_TIES_JSON
    names a file."""
    try:
        from tests import helpers
    except Exception:
        return
    tot = helpers.near_tie_summary()
    if tot is None:
        return
    terminalreporter.write_line(
        f"near-ties: {tot['requests']} sampled requests compared in {tot['tests']} checks; "
        f"excused {tot['excused_accept']} acceptance + {tot['excused_sample']} draw near-ties; "
        f"unexcused {tot['unexcused']}; smallest residual mass R {tot['min_residual_R']:.3g}")
    path = os.environ.get("NEAR_TIES_JSON")
    if path:
        import json
        rec = {"total": tot, "per_check": helpers.NEAR_TIES}
        with open(path, "w") as f:
            json.dump(rec, f, indent=1, default=float)
