import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    config.addinivalue_line("markers", "expects_timeout: the test makes a bounded dQ wait run out on purpose")


@pytest.fixture(autouse=True)
def _no_expired_waits(request):
    """Every GPU test must finish without a bounded wait running out (any call, not just the last)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import deterministic_attention_backward_amd as dab

    dab.wait_timeouts(reset=True)
    yield
    n = dab.wait_timeouts(reset=True)
    if request.node.get_closest_marker("expects_timeout") is None:
        assert n == 0, f"{n} bounded waits ran out during {request.node.nodeid}"
