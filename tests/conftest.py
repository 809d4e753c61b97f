import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-shape test (minutes of host work)")


def _announce(item):
    # Name the case before any GPU work starts, flushed, so a run that ends
    # abruptly still says which test was running.
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-test] {item.nodeid}", flush=True)


def pytest_runtest_setup(item):
    _announce(item)


@pytest.fixture(scope="session")
def hip():
    """The HIP library binding; fails loudly when the GPU or library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    from bit_block_float_amd import hif4

    hif4.require_gpu()
    return hif4
