import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on the real stderr before it runs, so a run that
    dies inside a kernel still shows which case it was."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
