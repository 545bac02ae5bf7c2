"""Seeded random shapes through every entry point, against the oracle.

The other GPU tests pick their sizes by hand: the workloads' own, one
element either side of every launch-shape switch, ragged tails.  Here a
fixed generator draws sizes log-uniformly over the whole range those
switches sit in (mostly 2^10 to 2^26 elements, a few below), peer counts
from 1 to 16, both formats and both output types, so that shape choices no
hand-picked case lands on
(a tile count just under a tail threshold, a grid one workgroup over an XCD
run) are compared with the oracle too.  Every output is compared: codes,
scales and E8M0 bytes bit for bit, sums bit for bit (which implies the 1e-6
gate).  Inputs come from the seeded generators; the oracle never takes one
from the HIP path."""
import numpy as np
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
import oracle
from dequantize_reduce_transfer_amd import workloads
from gpu_util import (assert_bf16_parity, assert_bytes_equal, dev_bf16, dev_f32, dev_u8,
                      f32_bits, host, require_gpu)

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(2026)


def _log_uniform(lo_bits, hi_bits, count):
    return [max(1, int(2.0 ** _RNG.uniform(lo_bits, hi_bits))) for _ in range(count)]


QUANT_CASES = [(n, int(_RNG.integers(0, 2)))
               for n in _log_uniform(0, 10, 3) + _log_uniform(10, 26.2, 13)]
REDUCE_CASES = []
for _n in _log_uniform(0, 10, 3) + _log_uniform(10, 26.5, 13):
    _k = int(_RNG.integers(1, 17))
    while _n * _k > (1 << 28):
        _n //= 2
    REDUCE_CASES.append((_n, _k, int(_RNG.integers(0, 2)), bool(_RNG.integers(0, 2))))
REQUANT_CASES = []
for _n in _log_uniform(0, 10, 2) + _log_uniform(10, 26.5, 10):
    _k = int(_RNG.integers(1, 17))
    while _n * _k > (1 << 28):
        _n //= 2
    REQUANT_CASES.append((_n, _k, int(_RNG.integers(0, 2)), int(_RNG.integers(0, 2))))
TW_CASES = [(n, int(_RNG.integers(0, 2))) for n in _log_uniform(0, 10, 1) + _log_uniform(10, 26, 5)]
MX_CASES = []
for _ in range(6):
    _K = 32 * int(_RNG.integers(1, 97))
    _rows = max(1, int(2.0 ** _RNG.uniform(10, 27.2)) // _K)
    _k = int(_RNG.integers(1, 5))
    while _rows * _K * _k > (1 << 27) and _rows > 1:
        _rows //= 2
    MX_CASES.append((_rows, _K, _k, bool(_RNG.integers(0, 2))))


def _planted_bits(n, seed):
    """A segmented gradient with a subnormal-range block, an inf, a NaN and
    a zero block planted at random block positions (where n allows)."""
    bits = workloads.bits(workloads.segmented_gradient(n, seed=seed, segment=1 << 16)).copy()
    nb = (n + 127) // 128
    rng = np.random.default_rng(seed)
    for kind in range(4):
        b = int(rng.integers(0, nb))
        lo, hi = 128 * b, min(n, 128 * b + 128)
        if kind == 0:
            bits[lo:hi] = np.arange(hi - lo, dtype=np.uint16) % 5
        elif kind == 1:
            bits[int(rng.integers(lo, hi))] = 0xFF80
        elif kind == 2:
            bits[int(rng.integers(lo, hi))] = 0x7FC3
        else:
            bits[lo:hi] = 0
    return bits


@pytest.mark.parametrize("n,fmt", QUANT_CASES, ids=["n%d-f%d" % c for c in QUANT_CASES])
def test_quantize_random_sizes(n, fmt):
    dev = require_gpu()
    bits = _planted_bits(n, seed=n % 9973)
    q, s = fq.fp8q_quantize(dev_bf16(bits, dev), fmt)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize(bits, fmt)
    assert_bytes_equal(host(q), q_o, "codes n=%d" % n)
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), "scales n=%d" % n)


def _wire(n, k, fmt, seed):
    shards = [workloads.random_wire_shard(n, seed=seed + p, fmt=fmt) for p in range(k)]
    return [a.numpy() for a, _ in shards], [b.numpy() for _, b in shards]


@pytest.mark.parametrize("n,k,fmt,bf16", REDUCE_CASES,
                         ids=["n%d-k%d-f%d-%s" % (c[0], c[1], c[2], "bf16" if c[3] else "f32")
                              for c in REDUCE_CASES])
def test_reduce_random_sizes(n, k, fmt, bf16):
    dev = require_gpu()
    qs, ss = _wire(n, k, fmt, seed=7000 + n % 997)
    out = torch.bfloat16 if bf16 else torch.float32
    y = fq.fp8q_dequant_reduce([dev_u8(a, dev) for a in qs], [dev_f32(b, dev) for b in ss], fmt,
                               out_dtype=out)
    torch.cuda.synchronize()
    want = oracle.dequant_reduce(qs, ss, fmt, out_bf16=bf16)
    if bf16:
        assert_bf16_parity(host(y), want, "reduce n=%d k=%d" % (n, k))
    else:
        assert_bytes_equal(f32_bits(host(y)), f32_bits(want), "reduce n=%d k=%d" % (n, k))


@pytest.mark.parametrize("n,k,fin,fout", REQUANT_CASES,
                         ids=["n%d-k%d-f%d%d" % c for c in REQUANT_CASES])
def test_requantize_random_sizes(n, k, fin, fout):
    dev = require_gpu()
    qs, ss = _wire(n, k, fin, seed=8000 + n % 991)
    q, s = fq.fp8q_dequant_reduce_requantize([dev_u8(a, dev) for a in qs],
                                             [dev_f32(b, dev) for b in ss], fin, fout)
    torch.cuda.synchronize()
    q_o, s_o = oracle.reduce_requantize(qs, ss, fin, fout)
    assert_bytes_equal(host(q), q_o, "requantize codes n=%d k=%d" % (n, k))
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), "requantize scales n=%d k=%d" % (n, k))


@pytest.mark.parametrize("rows,K,k,bf16", MX_CASES,
                         ids=["r%d-K%d-k%d-%s" % (c[0], c[1], c[2], "bf16" if c[3] else "f32")
                              for c in MX_CASES])
def test_mx8_random_shapes(rows, K, k, bf16):
    """The MXFP8 quantize of a [rows, K] weight, then the receiver's k-peer
    reduce of k such weights' oracle-made codes and E8M0 bytes."""
    dev = require_gpu()
    ws = [workloads.bits(workloads.kaiming_uniform((rows, K), seed=60 + p)).reshape(rows, K)
          for p in range(k)]
    q, e = fq.mx8_quantize(dev_bf16(ws[0], dev).view(rows, K))
    torch.cuda.synchronize()
    made = [oracle.mx8_quantize(w) for w in ws]
    assert_bytes_equal(host(q), made[0][0], "mx8 codes %dx%d" % (rows, K))
    assert_bytes_equal(host(e), made[0][1], "mx8 e8m0 %dx%d" % (rows, K))
    out = torch.bfloat16 if bf16 else torch.float32
    y = fq.mx8_dequant_reduce([dev_u8(a, dev).view(rows, K) for a, _ in made],
                              [dev_u8(b, dev).view(rows, K // 32) for _, b in made],
                              out_dtype=out)
    torch.cuda.synchronize()
    want = oracle.mx8_dequant_reduce([a for a, _ in made], [b for _, b in made], out_bf16=bf16)
    if bf16:
        assert_bf16_parity(host(y), want, "mx receiver %dx%d k=%d" % (rows, K, k))
    else:
        got, w = np.asarray(host(y), np.float32).ravel(), np.asarray(want, np.float32).ravel()
        assert np.array_equal(np.isnan(got), np.isnan(w)), "mx receiver NaN positions"
        ok = ~np.isnan(w)
        assert_bytes_equal(f32_bits(got[ok]), f32_bits(w[ok]), "mx receiver %dx%d k=%d" % (rows, K, k))


@pytest.mark.parametrize("n,fmt", TW_CASES, ids=["n%d-f%d" % c for c in TW_CASES])
def test_tensorwise_random_sizes(n, fmt):
    """The tensorwise quantize (one scale for the whole tensor) on a
    segmented gradient whose segments span six decades of scale."""
    dev = require_gpu()
    bits = workloads.bits(workloads.segmented_gradient(n, seed=n % 8191, segment=1 << 16))
    q, s = fq.fp8q_quantize_tensorwise(dev_bf16(bits, dev), fmt)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_tensorwise(bits, fmt)
    assert_bytes_equal(host(q), q_o, "tensorwise codes n=%d" % n)
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), "tensorwise scale n=%d" % n)
