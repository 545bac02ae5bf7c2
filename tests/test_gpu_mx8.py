"""GPU parity: MXFP8 weight quantize (HIP, through the C ABI) against the
oracle.  E4M3 codes and E8M0 scale bytes must match bit for bit."""
import numpy as np
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
import oracle
from brute_sets import mx_every_amax_rows
from dequantize_reduce_transfer_amd import workloads
from gpu_util import assert_bytes_equal, dev_bf16, host, require_gpu

pytestmark = pytest.mark.gpu


def _check(bits, dev, what):
    w = dev_bf16(bits, dev)
    q, e = fq.mx8_quantize(w)
    torch.cuda.synchronize()
    q_o, e_o = oracle.mx8_quantize(bits)
    assert tuple(q.shape) == q_o.shape and tuple(e.shape) == e_o.shape, what
    assert_bytes_equal(host(q), q_o, what + " codes")
    assert_bytes_equal(host(e), e_o, what + " e8m0")


def test_every_bf16_as_block_amax():
    dev = require_gpu()
    _check(mx_every_amax_rows(), dev, "every amax")


def test_bf16_natural_order():
    dev = require_gpu()
    _check(np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256), dev, "natural")


@pytest.mark.parametrize("name", ["gate", "up", "down"])
def test_moe_layer_shapes_four_experts(name):
    dev = require_gpu()
    layer = workloads.moe_layer(seed=0, experts=4)
    _check(workloads.bits(layer[name]).reshape(layer[name].shape), dev, name)


def test_k_equals_32_keeps_block_dim():
    dev = require_gpu()
    bits = workloads.bits(workloads.kaiming_uniform((37, 32), seed=4))
    w = dev_bf16(bits, dev).view(37, 32)
    q, e = fq.mx8_quantize(w)
    assert tuple(e.shape) == (37, 1)
    _check(bits.reshape(37, 32), dev, "K=32")


def test_3d_equals_flattened():
    dev = require_gpu()
    bits = workloads.bits(workloads.kaiming_uniform((5, 24, 96), seed=5)).reshape(5, 24, 96)
    w = dev_bf16(bits, dev).view(5, 24, 96)
    q3, e3 = fq.mx8_quantize(w)
    q2, e2 = fq.mx8_quantize(w.view(120, 96))
    assert torch.equal(q3.view(120, 96), q2) and torch.equal(e3, e2)
    _check(bits, dev, "3-D")


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 96), (7, 160), (64, 2048), (129, 768),
                                    (1000, 64), (2048 + 5, 128)])
def test_ragged_shapes_leave_canaries(rows, K):
    dev = require_gpu()
    rng = np.random.default_rng(rows * K)
    f = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-40, 40, (rows, 1)))).astype(np.float32)
    bits = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = dev_bf16(bits, dev).view(rows, K)
    n, nb = rows * K, rows * K // 32
    q_big = torch.full((n + 48,), 0x3C, dtype=torch.uint8, device=dev)
    e_big = torch.full((nb + 48,), 0xC3, dtype=torch.uint8, device=dev)
    fq.mx8_quantize(w, q_out=q_big[:n].view(rows, K), e8m0_out=e_big[:nb].view(rows, K // 32))
    torch.cuda.synchronize()
    q_o, e_o = oracle.mx8_quantize(bits)
    qh, eh = host(q_big), host(e_big)
    assert_bytes_equal(qh[:n], q_o, "codes")
    assert_bytes_equal(eh[:nb], e_o, "e8m0")
    assert np.all(qh[n:] == 0x3C) and np.all(eh[nb:] == 0xC3)


def test_zero_tiny_and_nonfinite_blocks():
    dev = require_gpu()
    w = np.zeros((4, 128), np.uint16)
    w[0, 5] = 0x3F80
    w[1, 40] = 0x0001             # bf16 subnormal amax
    w[1, 70] = 0x8080             # -2^-126
    w[2, 33] = 0x7F80             # +inf
    w[2, 99] = 0xFFC0             # NaN
    w[3, :32] = 0x8000            # -0 block
    w[3, 64] = 0x7F7F             # bf16 max
    w[3, 65] = 0x43E0             # 448
    w[3, 96] = 0x43F0             # 480: saturates
    _check(w, dev, "special blocks")


@pytest.mark.parametrize("offset", [1, 2, 3, 4])
def test_scale_pointer_at_any_byte_offset(offset):
    """E8M0 output at a pointer that is not 4-byte aligned (the kernel then
    writes its staged scale bytes one by one); bytes around it untouched."""
    dev = require_gpu()
    rows, K = 300, 2048                          # several workgroups of scale bytes
    w = workloads.kaiming_uniform((rows, K), seed=30 + offset, device=dev)
    ne = rows * K // 32
    buf = torch.full((ne + 8,), 0xA5, dtype=torch.uint8, device=dev)
    e = buf[offset:offset + ne]
    q, _ = fq.mx8_quantize(w, e8m0_out=e)
    torch.cuda.synchronize()
    q_o, e_o = oracle.mx8_quantize(workloads.bits(w).reshape(rows, K))
    assert_bytes_equal(host(q).ravel(), q_o.ravel(), "codes")
    b = host(buf)
    assert_bytes_equal(b[offset:offset + ne], e_o.ravel(), "e8m0")
    assert np.all(b[:offset] == 0xA5) and np.all(b[offset + ne:] == 0xA5)


@pytest.mark.parametrize("offset", [1, 4])
def test_scale_pointer_at_byte_offsets_one_wave_shape(offset):
    """The same on the one-wave shape (from 2^27 elements, ending with
    one-tile waves): [2^16 + 3, 2048] weights, E8M0 output at byte offsets
    1 and 4 between canaries, sampled rows (the first, the last and random
    ones) against the oracle."""
    dev = require_gpu()
    rows, K = (1 << 16) + 3, 2048
    w = workloads.kaiming_uniform((rows, K), seed=40 + offset, device=dev)
    ne = rows * K // 32
    buf = torch.full((ne + 8,), 0xA5, dtype=torch.uint8, device=dev)
    q, _ = fq.mx8_quantize(w, e8m0_out=buf[offset:offset + ne])
    torch.cuda.synchronize()
    e = buf[offset:offset + ne].view(rows, K // 32)
    rng = np.random.default_rng(offset)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(rows - 64, rows),
                                    rng.integers(0, rows, 2048)]))
    it = torch.from_numpy(idx).to(dev)
    q_o, e_o = oracle.mx8_quantize(host(w[it]))
    assert_bytes_equal(host(q[it]), q_o, "codes")
    assert_bytes_equal(host(e[it]), e_o, "e8m0")
    b = host(buf)
    assert np.all(b[:offset] == 0xA5) and np.all(b[offset + ne:] == 0xA5)


@pytest.mark.parametrize("rows", [2047, 2048])
def test_small_launch_switch_sizes(rows):
    """Below 2^22 elements the MXFP8 quantize takes one tile of one load per
    wave: [2047, 2048] and [2048, 2048] weights, every code and E8M0 byte
    against the oracle."""
    dev = require_gpu()
    K = 2048
    w = workloads.kaiming_uniform((rows, K), seed=rows, device=dev)
    _check(workloads.bits(w).reshape(rows, K), dev, "rows=%d" % rows)


@pytest.mark.parametrize("rows", [(1 << 16) - 1, 1 << 16])
def test_shape_switch_sizes(rows):
    """The MXFP8 launch changes shape at 2^27 elements (one-wave workgroups
    whose last 4096 tiles go one per wave): [rows, 2048] weights either
    side of it, sampled rows (the first, the last and random ones) against
    the oracle."""
    dev = require_gpu()
    K = 2048
    w = workloads.kaiming_uniform((rows, K), seed=rows % 13, device=dev)
    q, e = fq.mx8_quantize(w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(rows)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(rows - 64, rows),
                                    rng.integers(0, rows, 2048)]))
    it = torch.from_numpy(idx).to(dev)
    q_o, e_o = oracle.mx8_quantize(host(w[it]))
    assert_bytes_equal(host(q[it]), q_o, "codes rows=%d" % rows)
    assert_bytes_equal(host(e[it]), e_o, "e8m0 rows=%d" % rows)
