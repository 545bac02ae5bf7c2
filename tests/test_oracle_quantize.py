"""Pins for the oracle's block-128 quantize, dequantize and dequant-reduce.

Each check derives the expected value by another route than the oracle's own
code: numpy's IEEE fp32 division and reshaping for the per-block amax and
scale, torch's FP8 dtypes for decoding, the exact-rational nearest-code
search for rounding, closed forms (the pages' 48.4%, the largest element
landing on the largest code), and invariants (power-of-two scaling, sign
symmetry, error bounds, exact cancellation).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dequantize_reduce_transfer_amd import workloads
from exact_fp8 import nearest_codes
from helpers import (bf16_bits_to_f32, f32_to_bf16_bits, finite_bf16_patterns,
                     same_bits_bf16, same_bits_f32, torch_fp8_decode)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MAXV = {0: 448.0, 1: 57344.0}
MAX_CODE = {0: 0x7E, 1: 0x7B}
SMIN = np.float32(2.0 ** -126)


def _page_figure(name):
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line and line[0] == name:
                return float(line[1])
    raise KeyError(name)


def _np_blocks(xf, block=128):
    """Pad to whole blocks with zeros (zeros never change an amax)."""
    nb = (xf.size + block - 1) // block
    pad = np.zeros(nb * block, dtype=np.float32)
    pad[:xf.size] = xf
    return pad.reshape(nb, block)


def _expected_scales(xf, fmt):
    amax = np.abs(_np_blocks(xf)).max(axis=1).astype(np.float32)
    s = amax / np.float32(MAXV[fmt])          # numpy: IEEE fp32 division
    return np.maximum(s, SMIN)


def _tiny_bits(seed=0, n=1 << 16):
    return workloads.bits(workloads.tiny_gradient(seed, n=n, zero_block=3))


# --------------------------------------------------------------------------- #

def test_wire_bytes_match_page_figure():
    n = 128 * 1000
    q, s = oracle.quantize(np.zeros(n, np.uint16), oracle.E4M3)
    reduction = 100.0 * (1.0 - (q.nbytes + s.nbytes) / (2.0 * n))
    assert reduction == 48.4375
    assert round(reduction, 1) == _page_figure("wire_reduction_percent")
    qm, e = oracle.mx8_quantize(np.zeros((10, 3200), np.uint16))
    red_mx = 100.0 * (1.0 - (qm.nbytes + e.nbytes) / (2.0 * qm.size))
    assert round(red_mx, 1) == _page_figure("wire_reduction_percent")
    assert qm.nbytes / e.nbytes == _page_figure("mx_weight_to_scale_bytes")


@pytest.mark.parametrize("fmt", [0, 1])
def test_scales_are_block_amax_over_max(fmt):
    xb = _tiny_bits(1)
    xf = bf16_bits_to_f32(xb)
    q, s = oracle.quantize(xb, fmt)
    assert s.shape == ((xb.size + 127) // 128,)
    assert same_bits_f32(s, _expected_scales(xf, fmt))


@pytest.mark.parametrize("fmt", [0, 1])
def test_largest_element_takes_largest_code(fmt):
    xb = _tiny_bits(2)
    xf = bf16_bits_to_f32(xb)
    q, s = oracle.quantize(xb, fmt)
    blocks = _np_blocks(xf)
    qb = q.reshape(blocks.shape)
    for b in range(blocks.shape[0]):
        a = np.abs(blocks[b])
        if a.max() == 0:
            assert np.all((qb[b] & 0x7F) == 0)
            continue
        i = int(np.argmax(a))
        want = MAX_CODE[fmt] | (0x80 if blocks[b, i] < 0 else 0)
        assert qb[b, i] == want, b


@pytest.mark.parametrize("fmt", [0, 1])
def test_codes_are_nearest_to_fp32_quotient(fmt):
    """q_i = nearest FP8 code (rational search) to fl32(x_i / s_b) (numpy)."""
    xb = _tiny_bits(3, n=128 * 40 + 77)
    xf = bf16_bits_to_f32(xb)
    q, s = oracle.quantize(xb, fmt)
    s_rep = np.repeat(_expected_scales(xf, fmt), 128)[: xf.size]
    quot = xf / s_rep                           # IEEE fp32 division, elementwise
    assert np.array_equal(q, nearest_codes(quot, fmt))


def test_zero_block():
    xb = workloads.bits(workloads.tiny_gradient(0, n=1 << 20))
    q, s = oracle.quantize(xb, oracle.E4M3)
    zb = workloads.TINY_ZERO_BLOCK
    assert np.all(xb[zb * 128:(zb + 1) * 128] == 0)
    assert s[zb] == SMIN
    assert np.all(q[zb * 128:(zb + 1) * 128] == 0)
    y = oracle.dequantize(q, s, oracle.E4M3)
    assert np.all(y[zb * 128:(zb + 1) * 128] == 0)
    assert not np.any(np.isnan(y))


@pytest.mark.parametrize("fmt", [0, 1])
def test_negative_zero_block_keeps_signs(fmt):
    xb = np.full(128, 0x8000, np.uint16)
    xb[5] = 0
    q, s = oracle.quantize(xb, fmt)
    assert s[0] == SMIN
    want = np.full(128, 0x80, np.uint8)
    want[5] = 0
    assert np.array_equal(q, want)


@pytest.mark.parametrize("n", [1, 2, 96, 127, 129, 255, 256, 1000])
def test_partial_last_block_uses_only_valid_elements(n):
    rng = np.random.default_rng(n)
    xb = f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    q, s = oracle.quantize(xb, oracle.E4M3)
    assert q.shape == (n,) and s.shape == ((n + 127) // 128,)
    xf = bf16_bits_to_f32(xb)
    assert same_bits_f32(s, _expected_scales(xf, 0))
    # the tail block alone, as its own tensor, gives the same codes and scale
    lo = (n - 1) // 128 * 128
    q2, s2 = oracle.quantize(xb[lo:], oracle.E4M3)
    assert np.array_equal(q2, q[lo:]) and s2[0] == s[-1]


@pytest.mark.parametrize("fmt", [0, 1])
def test_power_of_two_invariance(fmt):
    """Scaling x by 2^j keeps every code and scales every scale by 2^j."""
    xf = bf16_bits_to_f32(_tiny_bits(4))
    q0, s0 = oracle.quantize(f32_to_bf16_bits(xf), fmt)
    for j in (-20, -3, 5, 30):
        xj = (xf.astype(np.float64) * 2.0 ** j).astype(np.float32)
        qj, sj = oracle.quantize(f32_to_bf16_bits(xj), fmt)
        assert np.array_equal(qj, q0), j
        live = s0 > SMIN                       # zero blocks keep the 2^-126 floor
        assert np.all(sj[~live] == SMIN)
        assert same_bits_f32(sj[live], (s0[live].astype(np.float64) * 2.0 ** j).astype(np.float32)), j


@pytest.mark.parametrize("fmt", [0, 1])
def test_sign_symmetry(fmt):
    xb = _tiny_bits(5)
    q0, s0 = oracle.quantize(xb, fmt)
    q1, s1 = oracle.quantize(xb ^ 0x8000, fmt)
    assert same_bits_f32(s0, s1)
    assert np.array_equal(q1, q0 ^ 0x80)


@pytest.mark.parametrize("fmt", [0, 1])
def test_roundtrip_error_bound(fmt):
    """|x - dec(q) s| <= 2^-(mbits+1) |x| (+ the fp32 quotient rounding) for
    quotients in the normal FP8 range, and <= half an FP8 subnormal step x s
    below it."""
    xb = _tiny_bits(6)
    xf = bf16_bits_to_f32(xb).astype(np.float64)
    q, s = oracle.quantize(xb, fmt)
    s_rep = np.repeat(s.astype(np.float64), 128)[: xf.size]
    back = torch_fp8_decode(q, fmt).astype(np.float64) * s_rep
    err = np.abs(back - xf)
    mbits = 3 if fmt == 0 else 2
    min_normal = 2.0 ** (-6 if fmt == 0 else -14)
    sub_step = 2.0 ** (-9 if fmt == 0 else -16)
    normal = np.abs(xf) / s_rep >= min_normal
    bound_n = 2.0 ** -(mbits + 1) * np.abs(xf) * (1 + 2.0 ** -20)
    assert np.all(err[normal] <= bound_n[normal])
    assert np.all(err[~normal] <= 0.5 * sub_step * s_rep[~normal] * (1 + 2.0 ** -20))


@pytest.mark.parametrize("fmt", [0, 1])
def test_nonfinite_block_policy(fmt):
    x = np.zeros(384, np.uint16)
    x[130] = 0x7F80          # +inf in block 1
    x[300] = 0xFFC1          # NaN in block 2
    x[5] = 0x3F80            # 1.0 in block 0
    q, s = oracle.quantize(x, fmt)
    assert s[0] == np.float32(1.0) / np.float32(MAXV[fmt])
    assert np.isnan(s[1]) and np.isnan(s[2])
    assert s[1:].view(np.uint32).tolist() == [0x7FC00000, 0x7FC00000]
    assert np.all(q[128:] == 0x7F)
    assert q[5] == MAX_CODE[fmt]


@pytest.mark.parametrize("fmt", [0, 1])
def test_single_value_blocks_every_bf16(fmt):
    """Each finite bf16 value alone in a block of zeros lands on +-max code
    (or +-0 for zero) and its scale is |v|/M, floored at 2^-126."""
    v = finite_bf16_patterns()
    x = np.zeros((v.size, 128), np.uint16)
    x[:, 17] = v
    q, s = oracle.quantize(x.ravel(), fmt)
    q = q.reshape(v.size, 128)
    vf = bf16_bits_to_f32(v)
    want_s = np.maximum(np.abs(vf) / np.float32(MAXV[fmt]), SMIN)
    assert same_bits_f32(s, want_s)
    sign = np.where(np.signbit(vf), 0x80, 0x00).astype(np.uint8)
    live = np.abs(vf) / np.float32(MAXV[fmt]) >= SMIN
    assert np.array_equal(q[live, 17], sign[live] | MAX_CODE[fmt])
    # below the scale floor the value is divided by 2^-126 (exact) and rounded
    floored = ~live
    assert np.array_equal(q[floored, 17], nearest_codes(vf[floored] * np.float32(2.0 ** 126), fmt))
    assert np.all(np.delete(q, 17, axis=1) == 0)


# --------------------------------------------------------------------------- #
# dequantize / dequant-reduce                                                  #
# --------------------------------------------------------------------------- #

def _lib_dequant(q, s, fmt):
    """torch decode x scale, both fp32 (one rounding), numpy repeat for the index."""
    return (torch_fp8_decode(q, fmt) * np.repeat(s, 128)[: q.size]).astype(np.float32)


@pytest.mark.parametrize("fmt", [0, 1])
def test_dequantize_matches_library_decode(fmt):
    q, s = workloads.random_wire_shard(128 * 50 + 33, seed=11, fmt=fmt)
    q, s = q.numpy(), s.numpy()
    want = _lib_dequant(q, s, fmt)
    assert same_bits_f32(oracle.dequantize(q, s, fmt), want)
    want_bf = f32_to_bf16_bits(want)
    assert same_bits_bf16(oracle.dequantize(q, s, fmt, out_bf16=True), want_bf)


@pytest.mark.parametrize("fmt", [0, 1])
def test_dequantize_all_codes_all_nan(fmt):
    q = np.tile(np.arange(256, dtype=np.uint8), 2)
    s = np.array([1.0, np.nan, 0.5, 3.0], np.float32)
    y = oracle.dequantize(q, s, fmt)
    assert same_bits_f32(y[:128], torch_fp8_decode(q[:128], fmt))
    assert np.all(np.isnan(y[128:256]))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("k", [1, 2, 4, 8, 16])
def test_reduce_is_ordered_fp32_sum(fmt, k):
    n = 128 * 24 + 5
    shards = [workloads.random_wire_shard(n, seed=100 + p, fmt=fmt) for p in range(k)]
    qs = [a.numpy() for a, _ in shards]
    ss = [b.numpy() for _, b in shards]
    acc = _lib_dequant(qs[0], ss[0], fmt)
    for p in range(1, k):
        acc = (acc + _lib_dequant(qs[p], ss[p], fmt)).astype(np.float32)
    got = oracle.dequant_reduce(qs, ss, fmt)
    assert same_bits_f32(got, acc)
    got_bf = oracle.dequant_reduce(qs, ss, fmt, out_bf16=True)
    assert same_bits_bf16(got_bf, f32_to_bf16_bits(acc))


@pytest.mark.parametrize("fmt", [0, 1])
def test_reduce_k1_is_dequantize(fmt):
    q, s = workloads.random_wire_shard(1000, seed=3, fmt=fmt)
    q, s = q.numpy(), s.numpy()
    q[:4] = [0x00, 0x80, 0x01, 0x81]
    assert same_bits_f32(oracle.dequant_reduce([q], [s], fmt), oracle.dequantize(q, s, fmt))


@pytest.mark.parametrize("fmt", [0, 1])
def test_reduce_cancels_exactly(fmt):
    xb = _tiny_bits(8)
    q0, s0 = oracle.quantize(xb, fmt)
    q1, s1 = oracle.quantize(xb ^ 0x8000, fmt)
    y = oracle.dequant_reduce([q0, q1], [s0, s1], fmt)
    assert np.all(y == 0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_reduce_within_fp32_bound_of_exact_sum(fmt):
    k, n = 8, 128 * 16
    xs = [workloads.bits(workloads.tiny_gradient(p, n=n, zero_block=None)) for p in range(k)]
    qs, ss = zip(*[oracle.quantize(x, fmt) for x in xs])
    got = oracle.dequant_reduce(list(qs), list(ss), fmt).astype(np.float64)
    terms = [torch_fp8_decode(q, fmt).astype(np.float64) * np.repeat(s, 128).astype(np.float64)
             for q, s in zip(qs, ss)]
    for i in range(0, n, 37):
        exact = sum(Fraction(float(t[i])) for t in terms)
        mag = sum(abs(float(t[i])) for t in terms)
        # each product and each of the k-1 additions rounds once in fp32
        assert abs(Fraction(float(got[i])) - exact) <= Fraction(k * 2.0 ** -24 * mag), i
