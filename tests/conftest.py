import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def gpu():
    """The HIP library on cuda:0; skips when this machine has no GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    import warp_specialized_gemm_amd as w  # raises if libwsg.so is missing
    torch.cuda.set_device(0)
    return w


def say(msg):
    """Flush a line naming the case before a GPU step."""
    print(msg, flush=True)
