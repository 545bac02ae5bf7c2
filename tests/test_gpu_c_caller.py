"""The C ABI used from C alone: tests/native/c_roundtrip.c allocates with
hipMalloc, creates its own HIP stream and passes host arrays of device
pointers; every output is checked against the C oracle."""
import os
import subprocess

import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "c_roundtrip.bin")


def test_c_caller_round_trip():
    require_gpu()
    if not os.path.exists(BIN):
        pytest.skip("the C caller is built by __graft_entry__.build()")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_roundtrip ok" in r.stdout
