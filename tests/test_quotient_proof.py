"""The block quantize kernel's divide-free quotient equals IEEE x / s.

Builds tests/native/quotient_exhaust.c with gcc (hardware fma, no
contraction) and runs its exhaustive check: every (bf16 significand,
fp32 scale significand) pair, every pair of bf16 exponents with every x
significand, and signed zeros.  The C file restates the kernel's per-element
formula from quantize.hip; it shares no code with the kernel or the oracle.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_markstein_quotient_is_correctly_rounded(tmp_path):
    exe = str(tmp_path / "quotient_exhaust")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "native", "quotient_exhaust.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches: 0" in r.stdout
