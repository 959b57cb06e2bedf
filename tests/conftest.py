import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _announce(request):
    """Name each test on the real stderr before it runs, so a GPU fault that
    ends the process still shows which case was running."""
    sys.__stderr__.write(f"\n[start] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
