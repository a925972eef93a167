import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _name_the_case(request):
    # a GPU run that dies takes its output with it: say which case is running first
    if request.node.get_closest_marker("gpu"):
        print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
