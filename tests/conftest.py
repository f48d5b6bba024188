import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)
    return load


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Names each GPU case on stderr (flushed) before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
