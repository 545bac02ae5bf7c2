"""Build the HIP library ``libfp8q.so`` in-tree for gfx950 with hipcc.

    python -m dequantize_reduce_transfer_amd.build

Cross-compiles without a GPU.  Flags:
  * ``--offload-arch=gfx950``  MI355X (CDNA4);
  * ``-ffp-contract=off``      every fp32 multiply and add is rounded on its
                               own, as the codec's definition requires (fused
                               multiply-adds are written out where intended);
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``  keeps the compiler
                               from forming packed fp32 instructions;
  * ``-mllvm -amdgpu-kernarg-preload-count=16``  the kernels' leading
                               arguments arrive preloaded in SGPRs instead of
                               through a scalar load at wave start (gfx950
                               supports it; the code object keeps a
                               fallback prologue); measured 0.5-1% faster for
                               the block quantize at 16-64 MiB payloads;
  * fp32 denormals stay enabled (no flush-to-zero flag).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libfp8q.so")

SOURCES = ["quantize.hip", "dequant_reduce.hip", "mx8_quantize.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CXXFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libfp8q.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
