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


def stratified_rows(M, tile, seed=0):
    """Rows to check at full size: three in every `tile`-row block of the output.

    Each output tile row (one workgroup row of the launch) contributes its first
    row, its last row and one at an offset that moves by 101 rows (mod tile) from
    one tile row to the next. Over a launch the moving row falls in every
    consumer wave's row block and at every lane position of a fragment, and
    every row covers all tile columns, so every workgroup's output tile is
    compared somewhere.
    """
    import numpy as np
    out = set()
    for i in range((M + tile - 1) // tile):
        r0 = i * tile
        for r in (r0, r0 + tile - 1, r0 + (37 + 101 * i + seed) % tile):
            out.add(min(M - 1, r))
    return np.array(sorted(out), dtype=np.int64)
