import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(session, config, items):
    # Start the GPU runtime once, first, in a process that has no worker
    # threads yet (the oracle's OpenMP pool and the input generator's thread
    # pool start later).
    if any(item.get_closest_marker("gpu") for item in items):
        import torch
        if torch.cuda.is_available():
            torch.cuda.init()
            torch.empty(1, device="cuda")
            torch.cuda.synchronize()


@pytest.fixture(scope="session")
def oracle():
    from oracle import oracle as o
    o._load()
    return o
