"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; every
other test runs on the CPU only.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: a longer CPU test (still minutes at most)")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr (uncaptured, flushed) before it runs, so a
    run that dies on the GPU still says which case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write("\n[gpu case] %s\n" % request.node.nodeid)
        sys.__stderr__.flush()
    yield
