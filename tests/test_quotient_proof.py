"""The kernels' divide-free quotients equal the IEEE divide x / s.

Builds tests/native/quotient_exhaust.c with gcc (hardware fma, no
contraction) and runs its exhaustive check: every (bf16 significand,
fp32 scale significand) pair, every pair of bf16 exponents with every x
significand, and signed zeros.  The C file restates the kernel's per-element
formula from quantize.hip; it shares no code with the kernel or the oracle.
"""
import os
import subprocess


HERE = os.path.dirname(os.path.abspath(__file__))


def test_markstein_quotient_is_correctly_rounded(tmp_path):
    exe = str(tmp_path / "quotient_exhaust")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "native", "quotient_exhaust.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches: 0" in r.stdout


def _build(tmp_path, src, name, extra=()):
    exe = str(tmp_path / name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-mfma", "-ffp-contract=off", "-fno-fast-math",
                    *extra, "-o", exe, os.path.join(HERE, "native", src), "-lm"], check=True)
    return exe


def test_quotient_exhaustive_in_emulated_precisions(tmp_path):
    """The kernels' quotient of a dividend as precise as the divisor (one
    Markstein step from RN(x * RN(1/s))) equals RN(x / s) for every pair of
    p-bit significands, p = 8 .. 13, in emulated p-bit arithmetic, and so
    does a second step.  (p = 14 .. 16 also pass; they take minutes: build
    with -DPMIN=14 -DPMAX=16.)"""
    exe = _build(tmp_path, "markstein_emulate.c", "markstein_emulate")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("one-step mismatches=0") == 6
    assert r.stdout.count("two-step mismatches=0") == 6


def test_quotient_random_and_boundary_fp32(tmp_path):
    """The same one-step sequence in real fp32 (hardware fma) against the
    IEEE divide on random pairs and on pairs whose quotient sits next to an
    fp32 rounding boundary, plus signed zeros."""
    exe = _build(tmp_path, "quotient_f32_random.c", "quotient_f32_random")
    r = subprocess.run([exe, "20000000", "11"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches=0" in r.stdout


def test_divide_free_block_scale_exhaustive(tmp_path):
    """The kernels' block scale without a divide (RN(amax / 7) by one
    Markstein step from RN(1/7), then the power-of-two factor and the
    2^-126 clamp) equals max(RN(amax / M), 2^-126) for every finite
    non-negative fp32 amax, for M = 448 and 57344."""
    exe = _build(tmp_path, "scale_div7_exhaust.c", "scale_div7_exhaust", extra=("-fopenmp",))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches: 0" in r.stdout


def test_quotient_never_exceeds_the_unclamped_encode_range(tmp_path):
    """The block-scale kernels convert RN(x / s) with no clamp.  For every
    finite non-negative fp32 amax and s = max(RN(amax / M), 2^-126), the
    largest quotient of the block, RN(amax / s), is at most M (1 + 2^-23)
    (the next fp32 above M), for M = 448 and 57344; it reaches that value
    for some amax, so the device check of the unclamped conversion has to
    cover it (tests/test_gpu_helpers.py)."""
    exe = _build(tmp_path, "quotient_bound_exhaust.c", "quotient_bound_exhaust",
                 extra=("-fopenmp",))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "e4m3: amax values 2139095040, bound 43e00001, over: 0" in r.stdout
    assert "e5m2: amax values 2139095040, bound 47600001, over: 0" in r.stdout
    assert "over: 0\n" in r.stdout
