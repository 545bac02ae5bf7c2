"""Pins for the oracle's MXFP8 (E4M3 + E8M0 per 32 along K) weight quantize.

Checks by other routes than the oracle's code: the defining property of the
E8M0 exponent (the scaled block maximum lands in [256, 512), i.e. in E4M3's
top binade) checked with numpy's ldexp for every bf16 amax; the rational
nearest-code search for the element codes; layout facts from the pages
(scales [rows, K/32] even when K == 32, 3-D == flattened 2-D); and
idempotence of quantize -> dequantize -> quantize.
"""
import numpy as np
import pytest

import oracle
from dequantize_reduce_transfer_amd import workloads
from exact_fp8 import nearest_codes
from helpers import bf16_bits_to_f32, f32_to_bf16_bits, finite_bf16_patterns, torch_fp8_decode


def test_e8m0_property_every_bf16_amax():
    """Each finite bf16 value v as the amax of a [1, 32] row."""
    v = finite_bf16_patterns()
    w = np.zeros((v.size, 32), np.uint16)
    w[:, 9] = v
    q, e = oracle.mx8_quantize(w)
    assert e.shape == (v.size, 1)
    codes = e[:, 0].astype(np.int64)
    vf = np.abs(bf16_bits_to_f32(v)).astype(np.float64)
    nz = vf > 0
    scaled = np.ldexp(vf, -(codes - 127))
    above_clamp = codes > 0
    # unclamped blocks: the block maximum lands in [2^8, 2^9)
    sel = nz & above_clamp
    assert np.all((scaled[sel] >= 256.0) & (scaled[sel] < 512.0))
    # code 0 (2^-127, the clamp): zeros and every amax below 2^-118; the
    # scaled maximum then stays below 512 and is never pushed past the range
    assert np.all(vf[~above_clamp] < 2.0 ** -118)
    assert np.all(scaled[~above_clamp] < 512.0)
    exact_binade = (vf >= 2.0 ** -119) & (vf < 2.0 ** -118)
    assert np.all(codes[exact_binade] == 0)
    assert np.all(codes[~nz] == 0)
    assert codes.max() <= 254


def test_elements_are_nearest_codes_of_scaled_values():
    rng = np.random.default_rng(5)
    K = 96
    w = f32_to_bf16_bits((rng.standard_normal((40, K)) * np.exp(rng.uniform(-30, 30, (40, 1))))
                         .astype(np.float32))
    w[3, 32:64] = 0
    q, e = oracle.mx8_quantize(w)
    wf = bf16_bits_to_f32(w).astype(np.float64)
    X = np.repeat(e.astype(np.int64) - 127, 32, axis=1)
    want = nearest_codes(np.ldexp(wf, -X).astype(np.float32), 0)
    assert np.array_equal(q, want)
    assert e[3, 1] == 0 and np.all(q[3, 32:64] == 0)


def test_largest_element_code_in_top_binade():
    w = workloads.bits(workloads.kaiming_uniform((64, 2048), seed=1))
    q, e = oracle.mx8_quantize(w)
    qb = q.reshape(-1, 32)
    wb = np.abs(bf16_bits_to_f32(w).reshape(-1, 32))
    top = qb[np.arange(qb.shape[0]), wb.argmax(axis=1)] & 0x7F
    # 256 <= code value <= 448: E4M3 codes 0x78 .. 0x7E
    assert np.all((top >= 0x78) & (top <= 0x7E))


def test_k_equals_32_keeps_block_dimension():
    w = workloads.bits(workloads.kaiming_uniform((7, 32), seed=2))
    q, e = oracle.mx8_quantize(w)
    assert q.shape == (7, 32) and e.shape == (7, 1)


def test_3d_equals_flattened_2d():
    w = workloads.bits(workloads.kaiming_uniform((3, 16, 64), seed=3))
    q3, e3 = oracle.mx8_quantize(w)
    q2, e2 = oracle.mx8_quantize(w.reshape(48, 64))
    assert e3.shape == (48, 2)
    assert np.array_equal(q3.reshape(48, 64), q2) and np.array_equal(e3, e2)


def test_rejects_k_not_multiple_of_32():
    with pytest.raises(ValueError):
        oracle.mx8_quantize(np.zeros((2, 48), np.uint16))


def test_idempotent_roundtrip():
    w = workloads.bits(workloads.kaiming_uniform((32, 256), seed=4))
    q, e = oracle.mx8_quantize(w)
    X = np.repeat(e.astype(np.int64) - 127, 32, axis=1)
    back = np.ldexp(torch_fp8_decode(q, 0).astype(np.float64), X).astype(np.float32)
    back_bits = f32_to_bf16_bits(back)
    assert np.array_equal(bf16_bits_to_f32(back_bits), back)      # exact in bf16
    q2, e2 = oracle.mx8_quantize(back_bits)
    assert np.array_equal(q2, q) and np.array_equal(e2, e)


def test_saturation_between_448_and_512():
    # amax = 480 * 2^k lands at 480 after scaling -> saturates to 448 (0x7E)
    w = np.zeros((1, 32), np.uint16)
    w[0, 0] = f32_to_bf16_bits(np.array([480.0 * 2.0 ** -20], np.float32))[0]
    w[0, 1] = f32_to_bf16_bits(np.array([-500.0 * 2.0 ** -20], np.float32))[0]
    w[0, 2] = f32_to_bf16_bits(np.array([256.0 * 2.0 ** -20], np.float32))[0]
    q, e = oracle.mx8_quantize(w)
    assert e[0, 0] == 127 - 20
    assert q[0, 0] == 0x7E and q[0, 1] == 0xFE and q[0, 2] == 0x78


def test_nonfinite_block_policy():
    w = np.zeros((2, 64), np.uint16)
    w[0, 40] = 0xFF80        # -inf in block (0, 1)
    w[1, 3] = 0x7FC0         # NaN in block (1, 0)
    w[1, 40] = 0x3F80        # 1.0 in block (1, 1)
    q, e = oracle.mx8_quantize(w)
    assert e[0, 1] == 0xFF and e[1, 0] == 0xFF
    assert e[0, 0] == 0 and e[1, 1] == 127 - 8
    assert np.all(q[0, 32:] == 0x7F) and np.all(q[1, :32] == 0x7F)
    assert np.all(q[0, :32] == 0)
    assert oracle.e8m0_decode(0xFF) != oracle.e8m0_decode(0xFF)      # NaN
    assert oracle.e8m0_decode(0) == 2.0 ** -127 and oracle.e8m0_decode(254) == 2.0 ** 127


def test_subnormal_bf16_amax_uses_its_true_exponent():
    # bf16 subnormal 0x0001 = 2^-133: floor(log2) = -133, X clamps to -127 and
    # the element scales to 2^-133 * 2^127 = 2^-6, E4M3's min normal (0x08).
    # bf16 normal 2^-100: X = -108, code 19, the element scales to 256 (0x78).
    w = np.zeros((2, 32), np.uint16)
    w[0, 0] = 0x0001
    w[1, 0] = f32_to_bf16_bits(np.array([2.0 ** -100], np.float32))[0]
    q, e = oracle.mx8_quantize(w)
    assert e[0, 0] == 0 and e[1, 0] == 19
    assert q[0, 0] == 0x08 and q[1, 0] == 0x78
    w[0, 0] = 0x0080                       # 2^-126 -> 2^1 = 2.0 (0x40)
    q, e = oracle.mx8_quantize(w)
    assert e[0, 0] == 0 and q[0, 0] == 0x40
