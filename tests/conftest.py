import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_report_header(config):
    return "biased full-graph attention: oracle pins (not gpu) and HIP parity (gpu)"


@pytest.fixture(autouse=True)
def _announce(request):
    # Name the case before it runs, so a run that ends abruptly still says where it was.
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
