"""Sizes whose grids hold several whole rounds of the XCD-aware workgroup
map plus a remainder that keeps the identity (and a ragged tail), checked in
full against the oracle: a wrong map would drop or repeat whole tiles."""
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
import oracle
from dequantize_reduce_transfer_amd import workloads
from gpu_util import (assert_bf16_parity, assert_bytes_equal, dev_f32, dev_u8, f32_bits, host,
                      require_gpu)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [9_000_333, 4_194_304 + 8192 * 77 + 5])
def test_quantize_many_rounds(n):
    dev = require_gpu()
    x = workloads.segmented_gradient(n, seed=n % 97, device=dev, segment=1 << 20)
    q, s = fq.fp8q_quantize(x, fq.E4M3)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize(workloads.bits(x), fq.E4M3)
    assert_bytes_equal(host(q), q_o, "codes n=%d" % n)
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), "scales n=%d" % n)


@pytest.mark.parametrize("k", [1, 3, 8, 9, 13, 14, 16])
def test_reduce_many_rounds(k):
    dev = require_gpu()
    n = 4_600_050
    shards = [workloads.random_wire_shard(n, seed=70 + p, fmt=fq.E4M3) for p in range(k)]
    qh = [a.numpy() for a, _ in shards]
    sh = [b.numpy() for _, b in shards]
    y = fq.fp8q_dequant_reduce([dev_u8(a, dev) for a in qh], [dev_f32(b, dev) for b in sh], fq.E4M3,
                               out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16_parity(host(y), oracle.dequant_reduce(qh, sh, fq.E4M3, out_bf16=True), "k=%d" % k)


@pytest.mark.parametrize("k", [2, 9, 12, 13, 16])
def test_requantize_many_rounds(k):
    dev = require_gpu()
    n = 4_600_050
    shards = [workloads.random_wire_shard(n, seed=90 + p, fmt=fq.E5M2) for p in range(k)]
    qh = [a.numpy() for a, _ in shards]
    sh = [b.numpy() for _, b in shards]
    q, s = fq.fp8q_dequant_reduce_requantize([dev_u8(a, dev) for a in qh],
                                             [dev_f32(b, dev) for b in sh], fq.E5M2, fq.E4M3)
    torch.cuda.synchronize()
    q_o, s_o = oracle.reduce_requantize(qh, sh, fq.E5M2, fq.E4M3)
    assert_bytes_equal(host(q), q_o, "codes k=%d" % k)
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), "scales k=%d" % k)


def test_mx8_many_rounds():
    dev = require_gpu()
    w = workloads.kaiming_uniform((4501, 2048), seed=8, device=dev)
    q, e = fq.mx8_quantize(w)
    torch.cuda.synchronize()
    q_o, e_o = oracle.mx8_quantize(workloads.bits(w).reshape(4501, 2048))
    assert_bytes_equal(host(q), q_o, "codes")
    assert_bytes_equal(host(e), e_o, "e8m0")
    y = fq.mx8_dequantize(q, e, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16_parity(host(y).ravel(), oracle.mx8_dequantize(q_o, e_o, out_bf16=True).ravel(),
                       "mx dequantize")


@pytest.mark.parametrize("k", [13, 16])
def test_requantize_one_wave_workgroups(k):
    """From 13 peers and 2^23 elements up the requantize runs one-wave
    workgroups in XCD runs of 256: this size holds two whole rounds of that
    map at k = 16, a remainder, and a ragged tail of 261 elements."""
    dev = require_gpu()
    n = (1 << 23) + 256 * 77 + 5
    shards = [workloads.random_wire_shard(n, seed=110 + p, fmt=fq.E4M3) for p in range(k)]
    qh = [a.numpy() for a, _ in shards]
    sh = [b.numpy() for _, b in shards]
    q, s = fq.fp8q_dequant_reduce_requantize([dev_u8(a, dev) for a in qh],
                                             [dev_f32(b, dev) for b in sh], fq.E4M3, fq.E4M3)
    torch.cuda.synchronize()
    q_o, s_o = oracle.reduce_requantize(qh, sh, fq.E4M3, fq.E4M3)
    assert_bytes_equal(host(q), q_o, "codes k=%d" % k)
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), "scales k=%d" % k)
