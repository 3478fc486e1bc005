import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle._load()
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU test on stderr (flushed) before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write("\n[gpu case] %s\n" % request.node.nodeid)
        sys.stderr.flush()
    yield


@pytest.fixture(scope="session")
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sliding_window_learnable_amd import _lib

    _lib.load()          # fails loudly if the HIP library is missing
    return torch.device("cuda:0")
