"""The CMake build (for C and C++ users) produces the same library: it
configures, compiles for gfx950 without a GPU, and exports every symbol the
header declares."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("cmake") is None or not os.path.exists("/opt/rocm/llvm/bin/clang++"),
                    reason="cmake or the ROCm compiler is not installed")
def test_cmake_builds_the_library(tmp_path):
    gen = ["-G", "Ninja"] if shutil.which("ninja") else []
    r = subprocess.run(["cmake", "-S", ROOT, "-B", str(tmp_path), *gen], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run(["cmake", "--build", str(tmp_path), "-j", "8"], capture_output=True,
                       text=True, timeout=1200)
    assert r.returncode == 0, r.stdout + r.stderr
    lib = tmp_path / "libfp8q.so"
    assert lib.exists()
    header = open(os.path.join(ROOT, "include", "fp8q.h")).read()
    declared = set(re.findall(r"^FP8Q_API [^(]*?\b(\w+)\s*\(", header, flags=re.M))
    out = subprocess.run(["nm", "-D", "--defined-only", str(lib)], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert declared and declared == exported
