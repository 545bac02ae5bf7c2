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


@pytest.fixture(scope="session", autouse=True)
def _built_libraries():
    """Build the HIP library (hipcc, no GPU needed) and the oracle if either is
    missing, so a fresh tree can run the suite; nothing is rebuilt otherwise."""
    import dequantize_reduce_transfer_amd as fq
    import oracle

    if not os.path.exists(fq.LIB_PATH) and not os.environ.get("FP8Q_LIB"):
        from dequantize_reduce_transfer_amd import build as hip_build
        sys.__stderr__.write("[conftest] building %s\n" % fq.LIB_PATH)
        hip_build.build()
    oracle.build(force=False)
    yield
