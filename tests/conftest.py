import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP path")


@pytest.fixture(scope="session")
def libqsa():
    """The HIP library; built in-tree only when nothing is built yet."""
    from block_sparse_long_amd import build, qsa
    if not os.path.exists(qsa.LIB_PATH):
        build.build()
    return qsa.load()


@pytest.fixture(scope="session")
def gpu(libqsa):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")
