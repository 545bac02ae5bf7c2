"""The kernels' divide-free helpers on the device, over every input they can
take: tests/native/helpers_exhaust.hip includes fp8q_device.h and compares
scale_from_amax (both formats, every finite non-negative fp32 amax) and
recip_rn (every normal x with a normal reciprocal) with hipcc's IEEE fp32
divide on the same GPU."""
import os
import subprocess

import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "helpers_exhaust.bin")


def test_divide_free_helpers_equal_ieee_divide_everywhere():
    require_gpu()
    if not os.path.exists(BIN):
        pytest.skip("the device check is built by __graft_entry__.build()")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches: 0" in r.stdout


QUOTIENT_BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native",
                            "quotient_f32_exhaust.bin")


def test_quotient_exhaustive_over_fp32_significands():
    """markstein_quotient (one Markstein step from RN(x * RN(1/s))) equals
    the IEEE divide for all 2^46 pairs of fp32 significands, x and s in
    [1, 2): with intermediates in the normal range every step scales exactly
    with x and s, so this covers every dividend (bf16 in the quantize, fp32
    in the requantize) and divisor the kernels can meet where the quotient
    can reach a nonzero FP8 code.  About 30 s."""
    require_gpu()
    if not os.path.exists(QUOTIENT_BIN):
        pytest.skip("the device check is built by __graft_entry__.build()")
    r = subprocess.run([QUOTIENT_BIN], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "pairs: 70368744177664" in r.stdout
    assert "mismatches: 0" in r.stdout
