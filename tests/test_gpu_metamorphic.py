"""Metamorphic properties checked on the GPU path itself (beyond parity):
scaling the input by a power of two keeps every code and scales the scales,
negating the input flips only sign bits, and rejected calls write nothing."""
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
from dequantize_reduce_transfer_amd import workloads
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2])
def test_power_of_two_scaling(fmt):
    dev = require_gpu()
    x = workloads.tiny_gradient(21, n=1 << 18, zero_block=None).to(dev)
    q0, s0 = fq.fp8q_quantize(x, fmt)
    for j in (-24, -3, 7, 40):
        xj = (x.float() * 2.0 ** j).to(torch.bfloat16)
        assert torch.equal(xj.float(), x.float() * 2.0 ** j)      # exact in bf16
        qj, sj = fq.fp8q_quantize(xj, fmt)
        assert torch.equal(qj, q0), j
        assert torch.equal(sj, s0 * 2.0 ** j), j


@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2])
def test_sign_symmetry(fmt):
    dev = require_gpu()
    x = workloads.tiny_gradient(22, n=(1 << 18) + 77).to(dev)
    q0, s0 = fq.fp8q_quantize(x, fmt)
    q1, s1 = fq.fp8q_quantize(-x, fmt)
    assert torch.equal(s0, s1)
    assert torch.equal(q1, q0 ^ 0x80)
    w = workloads.kaiming_uniform((64, 256), seed=5).to(dev)
    a, ea = fq.mx8_quantize(w)
    b, eb = fq.mx8_quantize(-w)
    assert torch.equal(ea, eb) and torch.equal(b, a ^ 0x80)


def test_rejected_calls_write_nothing():
    dev = require_gpu()
    L = fq.lib()
    n = 4096
    q = torch.zeros(n, dtype=torch.uint8, device=dev)
    s = torch.ones(n // 128, dtype=torch.float32, device=dev)
    y = torch.full((n,), 7.0, dtype=torch.float32, device=dev)
    qo = torch.full((n,), 0x11, dtype=torch.uint8, device=dev)
    so = torch.full((n // 128,), 3.0, dtype=torch.float32, device=dev)
    e = torch.zeros(n // 32, dtype=torch.uint8, device=dev)
    import ctypes
    PP = lambda *a: (ctypes.c_void_p * len(a))(*a)
    qa, sa = PP(q.data_ptr(), q.data_ptr()), PP(s.data_ptr(), s.data_ptr())
    assert L.fp8q_dequant_reduce(qa, sa, 2, n, 0, y.data_ptr(), 9, None) == 2          # bad dtype
    assert L.fp8q_dequant_reduce(qa, sa, 2, n, 0, y.data_ptr() + 4, 0, None) == 3      # misaligned
    assert L.fp8q_dequant_reduce_requantize(qa, sa, 2, n, 0, 0, qo.data_ptr(),
                                            so.data_ptr() + 1, None) == 3
    assert L.fp8q_dequant_reduce_requantize(qa, sa, 2, n, 0, 0, q.data_ptr(), so.data_ptr(), None) == 4
    assert L.mx8_dequantize(q.data_ptr(), e.data_ptr(), 128, 32, y.data_ptr(), 5, None) == 2
    assert L.fp8q_quantize_tensorwise(y.data_ptr(), n, 0, qo.data_ptr(), so.data_ptr() + 2, None) == 3
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and torch.all(qo == 0x11) and torch.all(so == 3.0)


def test_binding_rejects_wrong_output_sizes():
    """Output tensors of the wrong size are refused before any launch."""
    dev = require_gpu()
    n = 4096
    parts = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(3)]
    small = torch.full((n - 1,), 5.0, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        fq.fp8q_sum_f32(parts, out=small)
    q = torch.zeros(n, dtype=torch.uint8, device=dev)
    s = torch.ones(n // 128, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        fq.fp8q_dequant_reduce([q, q], [s, s], 0, out=small)
    with pytest.raises(ValueError):
        fq.fp8q_dequantize(q, s[:-1], 0)
    x = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        fq.fp8q_quantize(x, 0, q_out=q[:-16])
    torch.cuda.synchronize()
    assert torch.all(small == 5.0)
