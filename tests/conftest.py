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


def pytest_terminal_summary(terminalreporter):
    """Gradient checks of the run against both bars: the scale-relative one
    they assert, and the 2e-2 abs + 1e-2 rel bar of the outputs."""
    try:
        from tests.parity import GRAD_REPORT
    except Exception:
        return
    if not GRAD_REPORT:
        return
    tr = terminalreporter
    tr.write_sep("-", "gradient errors (%d checks)" % len(GRAD_REPORT))
    worst = {}          # per (gradient, dtype): the largest of each figure over its checks
    for what, dt, rel, bar, plain, abs_err, _rms in GRAD_REPORT:
        w = worst.setdefault((what, dt), [0.0, bar, 0.0, 0.0, 0])
        w[0], w[2], w[3] = max(w[0], rel), max(w[2], plain), max(w[3], abs_err)
        w[1] = max(w[1], bar)             # the loosest bar applied (per-case bars)
        w[4] += 1
    tr.write_line("%-6s %-9s %7s %14s %6s %19s %10s" % (
        "grad", "dtype", "checks", "err/(rms+|r|)", "bar", "err/(2e-2+1e-2|r|)", "max |err|"))
    for (what, dt), (rel, bar, plain, abs_err, n) in sorted(worst.items()):
        tr.write_line("%-6s %-9s %7d %14.3g %6.0e %19.3g %10.3g" % (
            what, dt, n, rel, bar, plain, abs_err))
