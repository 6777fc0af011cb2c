import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of host time")


def _ensure_host_libs():
    # The generator and the oracle are plain C++ built with g++; build them
    # if a fresh checkout has not been built yet.  The GPU library is never
    # built here: GPU tests load what __graft_entry__.build() produced.
    import oracle
    import synth
    for mod in (synth, oracle):
        if not os.path.exists(mod._LIB):
            mod.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def cuda_device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")
