"""GPU parity: block-128 quantize (HIP, through the C ABI) against the oracle.

FP8 codes and fp32 scales must match bit for bit.
"""
import numpy as np
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
import oracle
from brute_sets import b1_single_value_blocks, b2_natural_order, b3_anchor_sweep
from dequantize_reduce_transfer_amd import workloads
from gpu_util import assert_bytes_equal, dev_bf16, f32_bits, host, require_gpu

pytestmark = pytest.mark.gpu
FMTS = [fq.E4M3, fq.E5M2]


def _check_quantize(bits, fmt, dev, what):
    x = dev_bf16(bits, dev)
    q, s = fq.fp8q_quantize(x, fmt)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize(bits, fmt)
    assert_bytes_equal(host(q), q_o, what + " codes")
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), what + " scales")


@pytest.mark.parametrize("fmt", FMTS)
def test_tiny_gradient(fmt):
    dev = require_gpu()
    bits = workloads.bits(workloads.tiny_gradient(0))
    _check_quantize(bits, fmt, dev, "tiny seed 0")


@pytest.mark.parametrize("fmt", FMTS)
def test_b1_every_bf16_alone_in_a_block(fmt):
    dev = require_gpu()
    _check_quantize(b1_single_value_blocks(), fmt, dev, "B1")


@pytest.mark.parametrize("fmt", FMTS)
def test_b2_natural_order(fmt):
    dev = require_gpu()
    _check_quantize(b2_natural_order(), fmt, dev, "B2")


@pytest.mark.parametrize("fmt", FMTS)
def test_b3_anchor_sweep(fmt):
    dev = require_gpu()
    _check_quantize(b3_anchor_sweep(), fmt, dev, "B3")


@pytest.mark.parametrize("fmt", FMTS)
def test_stress_blocks(fmt):
    dev = require_gpu()
    bits = workloads.bits(workloads.stress_payload(5, fmt, n=1 << 20))
    _check_quantize(bits, fmt, dev, "stress")


RAGGED = [1, 2, 7, 8, 9, 96, 127, 128, 129, 255, 1000, 2047, 2048, 2049, 4173, 7144,
          65536 + 13, 3 * 2048 * 256 + 555]


@pytest.mark.parametrize("n", RAGGED)
@pytest.mark.parametrize("fmt", FMTS)
def test_ragged_sizes_leave_canaries(fmt, n):
    dev = require_gpu()
    rng = np.random.default_rng(n)
    f = (rng.standard_normal(n) * np.exp(rng.uniform(-8, 8, n))).astype(np.float32)
    bits = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nb = (n + 127) // 128
    x = dev_bf16(bits, dev)
    q_big = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device=dev)
    s_big = torch.full((nb + 16,), -7.0, dtype=torch.float32, device=dev)
    fq.fp8q_quantize(x, fmt, q_out=q_big[:n], scales_out=s_big[:nb])
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize(bits, fmt)
    qh, sh = host(q_big), host(s_big)
    assert_bytes_equal(qh[:n], q_o, "codes n=%d" % n)
    assert_bytes_equal(f32_bits(sh[:nb]), f32_bits(s_o), "scales n=%d" % n)
    assert np.all(qh[n:] == 0xA5), "codes written past n"
    assert np.all(sh[nb:] == -7.0), "scales written past the last block"


@pytest.mark.parametrize("fmt", FMTS)
def test_nonfinite_and_zero_blocks(fmt):
    dev = require_gpu()
    x = np.zeros(128 * 6 + 50, np.uint16)
    x[3] = 0x3F80
    x[128 + 9] = 0x7F80          # +inf
    x[256 + 1] = 0xFF80          # -inf
    x[384 + 100] = 0x7FC1        # NaN
    x[512:640] = 0x8000          # -0 block
    x[640 + 10] = 0xFFC0         # NaN in the partial block
    _check_quantize(x, fmt, dev, "non-finite")


def test_deterministic_and_stream_ordered():
    dev = require_gpu()
    bits = workloads.bits(workloads.tiny_gradient(1))
    x = dev_bf16(bits, dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q1, s1 = fq.fp8q_quantize(x, fq.E4M3)
        q2, s2 = fq.fp8q_quantize(x, fq.E4M3)
    s.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def test_failed_call_writes_nothing():
    dev = require_gpu()
    x = torch.ones(4096, dtype=torch.bfloat16, device=dev)
    q = torch.full((4096,), 0x5A, dtype=torch.uint8, device=dev)
    s = torch.full((32,), 3.0, dtype=torch.float32, device=dev)
    L = fq.lib()
    assert L.fp8q_quantize(x.data_ptr(), 4096, 7, q.data_ptr(), s.data_ptr(), None) == 2
    assert L.fp8q_quantize(x.data_ptr(), 4096, 0, q.data_ptr(), s.data_ptr() + 2, None) == 3
    assert L.fp8q_quantize(x.data_ptr(), 4096, 0, q.data_ptr(), q.data_ptr() + 64, None) == 4
    with pytest.raises(ValueError):
        fq.fp8q_quantize(x, 7, q_out=q, scales_out=s)
    torch.cuda.synchronize()
    assert torch.all(q == 0x5A) and torch.all(s == 3.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_outputs_at_odd_word_offsets(fmt):
    """scales_out only 4-byte aligned (odd word offsets): the workgroup's
    staged scales still land in place, and the words around them stay."""
    dev = require_gpu()
    n = 8192 * 37 + 300                          # several workgroup rounds and a tail
    nb = (n + 127) // 128
    x = workloads.segmented_gradient(n, seed=12, device=dev, segment=1 << 14)
    q_o, s_o = oracle.quantize(workloads.bits(x), fmt)
    for off in (1, 3):
        buf = torch.full((nb + off + 5,), -2.5, dtype=torch.float32, device=dev)
        q, s = fq.fp8q_quantize(x, fmt, scales_out=buf[off:off + nb])
        torch.cuda.synchronize()
        b = host(buf)
        assert_bytes_equal(host(q), q_o, "codes")
        assert_bytes_equal(f32_bits(b[off:off + nb]), f32_bits(s_o), "scales")
        assert np.all(b[:off] == -2.5) and np.all(b[off + nb:] == -2.5)


@pytest.mark.parametrize("n", [(1 << 23) + 77, (3 << 24) + 77])
def test_scale_outputs_at_odd_word_offsets_split_shapes(n):
    """The same on the launches that end with one-tile waves: the 4-wave
    shape (from 2^23 elements) and the one-wave shape (from 3 * 2^24), whose
    workgroups flush 64 and 16 scales per round."""
    dev = require_gpu()
    nb = (n + 127) // 128
    x = workloads.segmented_gradient(n, seed=13, device=dev, segment=1 << 20)
    q_o, s_o = oracle.quantize(workloads.bits(x), fq.E4M3)
    buf = torch.full((nb + 6,), -2.5, dtype=torch.float32, device=dev)
    q, s = fq.fp8q_quantize(x, fq.E4M3, scales_out=buf[1:1 + nb])
    torch.cuda.synchronize()
    b = host(buf)
    assert_bytes_equal(host(q), q_o, "codes")
    assert_bytes_equal(f32_bits(b[1:1 + nb]), f32_bits(s_o), "scales")
    assert b[0] == -2.5 and np.all(b[1 + nb:] == -2.5)


@pytest.mark.parametrize("n", [7168 * 512, 7168 * 512 + 1, (1 << 22) - 1, 1 << 22,
                               (1 << 23) - 1, (1 << 23) + 77,
                               (3 << 24) - 1, (3 << 24) + 77])
def test_shape_switch_sizes(n):
    """The launch shape changes at 2^22 elements (below, one tile of one
    load per wave; from there, two tiles of two loads), at 2^23 (a one-tile
    tail of 4096 tiles) and at 3 * 2^24 (one-wave workgroups): one element
    either side of each (ragged above), e5m2,
    every code and scale against the oracle.  A
    gradient with planted blocks near both ends -- bf16 subnormals (amax
    below 2^-60), an inf, a NaN, zeros -- so that waves take both the
    finite-and-normal path and the general one."""
    dev = require_gpu()
    x = workloads.segmented_gradient(n, seed=n % 101, device=dev, segment=1 << 20)
    bits = workloads.bits(x).copy()
    for base in (0, (n // 128 - 40) * 128):
        bits[base + 128 * 3:base + 128 * 4] = np.arange(128, dtype=np.uint16) % 7 | 0x8000 * (
            np.arange(128) % 2).astype(np.uint16)
        bits[base + 128 * 5 + 17] = 0x7F80
        bits[base + 128 * 7:base + 128 * 8] = 0
        bits[base + 128 * 9 + 100] = 0xFFC1
    _check_quantize(bits, fq.E5M2, dev, "n=%d" % n)
