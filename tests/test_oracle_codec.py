"""Pins for the oracle's FP8 codecs (CPU only).

The oracle's decoder and encoder are checked against things other than
themselves: the OCP spec constants (tests/golden), PyTorch's FP8 dtypes (a
library conversion), and an exact-rational brute-force nearest-value search.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_fp8 import nearest_code, nearest_codes
from helpers import all_bf16_patterns, bf16_bits_to_f32, same_bits_f32, torch_fp8_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMTS = {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2}
# Smallest magnitude at which torch's (non-saturating) cast leaves the finite
# range; below it, RNE to the format and satRNE agree.
TORCH_OVERFLOW = {oracle.E4M3: 464.0, oracle.E5M2: 61440.0}
MAX_CODE = {oracle.E4M3: 0x7E, oracle.E5M2: 0x7B}


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "ocp_fp8_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                fmt, code, val = line.split()
                rows.append((FMTS[fmt], int(code, 16), val))
    return rows


@pytest.mark.parametrize("fmt", [0, 1])
def test_decode_all_codes_match_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    assert same_bits_f32(oracle.fp8_decode(codes, fmt), torch_fp8_decode(codes, fmt))


def test_decode_spec_constants():
    rows = _golden_rows()
    assert len(rows) >= 20
    for fmt, code, val in rows:
        got = float(oracle.fp8_decode(np.array([code], np.uint8), fmt)[0])
        if val == "nan":
            assert math.isnan(got), (fmt, hex(code))
        elif val == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0
        else:
            want = float(val)
            assert got == want, (fmt, hex(code), got, want)
            if want == 0.0:
                assert math.copysign(1.0, got) > 0


def test_format_maxima():
    assert oracle.fp8_max(oracle.E4M3) == 448.0
    assert oracle.fp8_max(oracle.E5M2) == 57344.0


def _structured_f32():
    """fp32 values probing every rounding position: for each binade that
    reaches the FP8 range, all 256 combinations of the top 8 mantissa bits
    with a set of low-bit patterns (exact ties, just below/above ties,
    sticky bits), both signs."""
    top = np.arange(256, dtype=np.uint32) << 15
    low = np.array([0, 1, 0x3FFF, 0x4000, 0x4001, 0x7FFF, 0x2000, 0x5555], dtype=np.uint32)
    mant = (top[:, None] | low[None, :]).ravel()
    exps = np.arange(127 - 24, 127 + 18, dtype=np.uint32)     # 2^-24 .. 2^17
    bits = ((exps[:, None] << 23) | mant[None, :]).ravel()
    bits = np.concatenate([bits, bits | 0x80000000, np.arange(0, 1 << 12, dtype=np.uint32)])
    return bits.view(np.float32)


@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_matches_torch_cast_below_overflow(fmt):
    rng = np.random.default_rng(1234 + fmt)
    rand = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32).view(np.float32)
    ys = np.concatenate([_structured_f32(), rand, bf16_bits_to_f32(all_bf16_patterns())])
    ys = ys[np.isfinite(ys) & (np.abs(ys) < TORCH_OVERFLOW[fmt])]
    dt = torch.float8_e4m3fn if fmt == 0 else torch.float8_e5m2
    want = torch.from_numpy(ys).to(dt).view(torch.uint8).numpy()
    got = oracle.fp8_encode(ys, fmt)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(ys[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_saturates(fmt):
    m = oracle.fp8_max(fmt)
    big = np.array([TORCH_OVERFLOW[fmt], np.nextafter(np.float32(m), np.float32(np.inf)),
                    m * 1.5, m * 4, 3e38, np.inf], dtype=np.float32)
    assert np.all(oracle.fp8_encode(big, fmt) == MAX_CODE[fmt])
    assert np.all(oracle.fp8_encode(-big, fmt) == (0x80 | MAX_CODE[fmt]))
    nan = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(oracle.fp8_encode(nan, fmt) == 0x7F)
    assert oracle.fp8_encode(np.array([m], np.float32), fmt)[0] == MAX_CODE[fmt]


def test_encode_tie_examples():
    cases_e4m3 = [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
                  (464.0, 0x7E), (500.0, 0x7E), (-0.0, 0x80), (2.0 ** -9, 0x01),
                  (2.0 ** -6 - 2.0 ** -10, 0x08)]
    for v, c in cases_e4m3:
        assert oracle.fp8_encode_exact(v, oracle.E4M3) == c, v
    cases_e5m2 = [(61440.0, 0x7B), (57344.0, 0x7B), (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02),
                  (1.125, 0x3C), (1.375, 0x3E)]
    for v, c in cases_e5m2:
        assert oracle.fp8_encode_exact(v, oracle.E5M2) == c, v


@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_vs_exact_nearest_search(fmt):
    """All finite bf16 values times a few scales against the rational search."""
    b = all_bf16_patterns()
    v = bf16_bits_to_f32(b)
    v = v[np.isfinite(v)]
    rng = np.random.default_rng(7 + fmt)
    sel = np.concatenate([v[::7], rng.choice(v, 2000)])
    for scale in (1.0, 2.0 ** 8, 2.0 ** -8, 448.0 / 3.0, 1.0 / 57344.0):
        with np.errstate(over="ignore"):
            ys = (sel.astype(np.float64) * scale).astype(np.float32)
        want = nearest_codes(ys, fmt)
        got = oracle.fp8_encode(ys, fmt)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(float(ys[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_roundtrip_every_code(fmt):
    """Every finite code decodes to a value that encodes back to that code."""
    codes = np.arange(256, dtype=np.uint8)
    vals = torch_fp8_decode(codes, fmt)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.fp8_encode(vals[fin], fmt), codes[fin])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.integers(0, 1 << 32, size=1 << 16, dtype=np.uint64).astype(np.uint32).view(np.float32)
    # exact ties (low half 0x8000) on both even and odd upper halves, and
    # the values just either side of them
    hi = rng.integers(0, 0xFF7F, size=4096, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x17FFF, hi | 0x7FFF, hi | 0x8001]).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38], np.float32)])
    x = x[~np.isnan(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert oracle.f32_to_bf16(float("nan")) == 0x7FC0


def test_nearest_code_reference_is_sane():
    # the brute-force reference itself, on hand-checkable values
    assert nearest_code(448.0, 0) == 0x7E
    assert nearest_code(1.0, 0) == 0x38
    assert nearest_code(-1.0, 1) == 0xBC
    assert nearest_code(1e6, 1) == 0x7B
