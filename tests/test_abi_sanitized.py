"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU.

csrc/api.hip (argument validation and dispatch) is compiled host-only with
g++ and the sanitizers, and linked with tests/native/abi_stub_launchers.cpp
in place of the kernels: the stubs enqueue nothing, check the invariants a
validated call guarantees the launchers, and record each call.  Every case
of tests/test_abi.py then runs against that build in a child process with
the sanitizer runtime preloaded, including the accepted-call cases that only
the host-check build can run without a GPU.  Python's own allocator is switched to
malloc there so that a read past a short host array of peer pointers is a
sanitizer report rather than a silent read inside a Python arena, and the
child runs with pytest's output capture off, so that a sanitizer report that
ends the child still reaches this test's failure message.
"""
import os
import re
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "dequantize_reduce_transfer_amd", "csrc")


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_layer_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("sanitizer runtime not installed")
    lib = str(tmp_path / "libfp8q_hostcheck.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-fPIC", "-shared", "-o", lib,
           "-x", "c++", os.path.join(CSRC, "api.hip"),
           "-x", "none", os.path.join(HERE, "native", "abi_stub_launchers.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, FP8Q_LIB=lib, LD_PRELOAD=asan, PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"),
                        "-q", "-s", "-p", "no:cacheprovider", "-rs"],
                       capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    m = re.search(r"(\d+) passed", out)
    assert m and "skipped" not in out, out[-2000:]
