import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    """Name each test on the real stderr before it runs, so a run that ends
    abruptly still shows which case was on the GPU."""
    sys.__stderr__.write(f"[case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
