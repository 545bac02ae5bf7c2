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


CVT_BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "cvt_exhaust.bin")


def test_encode_step_equals_oracle_for_every_fp32():
    """The MXFP8 kernels' FP8 encode step -- clamp to +-FP8_MAX (sat_clamp),
    then the gfx950 packed conversion (cvt4) -- for all 2^32 fp32 patterns, the
    block-scale kernels' unclamped encode (cvt4 alone) for every fp32 in
    [-M (1 + 2^-23), M (1 + 2^-23)] (the range their quotients stay in),
    their fp32 -> bf16 output conversion (bf16_pack2) for all 2^32 fp32
    patterns, and the MXFP8 receiver's scaled decode (mx_dec2) for every
    E4M3 code and E8M0 scale, run on the device, each result compared on the
    host with the oracle (integer-exact satRNE in e4m3 and e5m2;
    round-to-nearest-even bf16; the oracle's MXFP8 dequantize).  NaN patterns (2 * (2^23 - 1)) are left out of the FP8 passes,
    since no kernel converts a NaN to FP8, and counted apart in the bf16
    pass.  About 25 s, mostly the oracle on the host's threads."""
    require_gpu()
    if not os.path.exists(CVT_BIN):
        pytest.skip("the device check is built by __graft_entry__.build()")
    r = subprocess.run([CVT_BIN], capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stdout + r.stderr
    nans = 2 * ((1 << 23) - 1)
    per_pass = (1 << 32) - nans
    for name in ("e4m3", "e5m2", "bf16"):
        assert "%s: compared %d fp32 patterns" % (name, per_pass) in r.stdout, r.stdout
    # the unclamped encode of the block-scale kernels on [-B, B], B = M (1 + 2^-23)
    unclamped = 0
    for name, bound in (("e4m3", 0x43E00001), ("e5m2", 0x47600001)):
        cnt = 2 * (bound + 1)
        assert ("%s unclamped: compared %d fp32 patterns in [-%08X, %08X], mismatches 0"
                % (name, cnt, bound, bound)) in r.stdout, r.stdout
        unclamped += cnt
    # the MXFP8 receiver's scaled decode: every code x every E8M0 scale, 4 positions
    assert "mx scaled decode: compared 262144 values" in r.stdout, r.stdout
    assert "NaN 3064, mismatches 0" in r.stdout, r.stdout
    assert "values: %d mismatches: 0" % (3 * per_pass + unclamped + 262144) in r.stdout, r.stdout
    assert "bf16 nan: %d NaN patterns" % nans in r.stdout, r.stdout
