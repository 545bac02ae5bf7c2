"""Every output at the full workload sizes, not a sample.

The oracle is too slow for 3.5e9 elements, so each full-size output is
checked against an independent restatement of the same rule in plain
PyTorch ops on the GPU (IEEE fp32 tensor-by-tensor divide, multiply and add
as separate kernels; a clamp to +-FP8_MAX and torch's round-to-nearest-even
float8 casts).  That torch checker is first pinned to the oracle, bit for bit, on
inputs that reach every rounding and saturation case (the stress payload
categories, every bf16 pattern as a block maximum), so a full-size match is
a match with the oracle's rule."""
import numpy as np
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
import oracle
from brute_sets import mx_every_amax_rows
from dequantize_reduce_transfer_amd import workloads
from gpu_util import dev_bf16, host, require_gpu

pytestmark = pytest.mark.gpu

FP8 = {fq.E4M3: torch.float8_e4m3fn, fq.E5M2: torch.float8_e5m2}
FMAX = {fq.E4M3: 448.0, fq.E5M2: 57344.0}
CHUNK = 1 << 27                                   # elements per checker pass


# ---------------------------------------------------------------- checkers --

def torch_quantize(x: torch.Tensor, fmt: int):
    """Block-128 rule on a finite bf16 chunk whose length is a multiple of 128."""
    xf = x.float().view(-1, 128)
    amax = xf.abs().amax(dim=1)
    # tensor / tensor: torch turns a division by a Python scalar into a
    # multiplication by its reciprocal on the GPU, which is not the IEEE divide
    s = torch.clamp(amax / torch.full_like(amax, FMAX[fmt]), min=2.0 ** -126)
    q = torch.clamp(xf / s[:, None], -FMAX[fmt], FMAX[fmt]).to(FP8[fmt])
    return q.view(torch.uint8).view(-1), s


def torch_reduce(qs, ss, fmt: int, a: int, b: int):
    """Ordered fp32 sum of the dequantized peers over elements [a, b) (a % 128 == 0)."""
    acc = None
    for q, s in zip(qs, ss):
        sc = s[a // 128:(b + 127) // 128].repeat_interleave(128)[:b - a]
        d = q[a:b].view(FP8[fmt]).float() * sc
        acc = d if acc is None else acc + d
    return acc


def torch_mx8(w: torch.Tensor):
    """MXFP8 rule on finite bf16 rows [rows, K]."""
    xf = w.float().view(-1, 32)
    amax = xf.abs().amax(dim=1)
    _, e = torch.frexp(amax)                      # amax = m * 2^e, m in [0.5, 1)
    X = torch.clamp(e.to(torch.int32) - 1 - 8, -127, 127)
    X = torch.where(amax == 0, torch.full_like(X, -127), X)
    mul = ((127 - X) << 23).view(torch.float32)   # 2^-X, a normal number for bf16 input
    q = torch.clamp(xf * mul[:, None], -448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).view(w.shape), (X + 127).to(torch.uint8).view(w.shape[0], -1)


def _mismatch(a: torch.Tensor, b: torch.Tensor) -> int:
    return int((a.view(-1) != b.view(-1)).sum().item())


# ------------------------------------------- the checker against the oracle --

@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2])
def test_torch_checker_equals_oracle(fmt):
    dev = require_gpu()
    x = workloads.stress_payload(7, fmt, n=1 << 20, device=dev)
    q_t, s_t = torch_quantize(x, fmt)
    q_o, s_o = oracle.quantize(workloads.bits(x), fmt)
    assert np.array_equal(host(q_t), q_o)
    assert np.array_equal(host(s_t).view(np.uint32), s_o.view(np.uint32))
    # every bf16 finite pattern as a value, in blocks with varied maxima
    allb = np.arange(0x10000, dtype=np.uint16)
    allb = allb[(allb & 0x7FFF) < 0x7F80]
    allb = allb[: allb.size // 128 * 128]
    xb = dev_bf16(np.random.default_rng(3).permutation(allb), dev)
    q_t, s_t = torch_quantize(xb, fmt)
    q_o, s_o = oracle.quantize(workloads.bits(xb), fmt)
    assert np.array_equal(host(q_t), q_o)
    assert np.array_equal(host(s_t).view(np.uint32), s_o.view(np.uint32))
    # the reduce
    shards = [workloads.random_wire_shard(128 * 4096 + 77, seed=9 + p, fmt=fmt, device=dev)
              for p in range(5)]
    qs = [a for a, _ in shards]
    ss = [b for _, b in shards]
    y_t = torch_reduce(qs, ss, fmt, 0, qs[0].numel())
    y_o = oracle.dequant_reduce([host(a) for a in qs], [host(b) for b in ss], fmt)
    assert np.array_equal(host(y_t).view(np.uint32), y_o.view(np.uint32))


def test_torch_mx_checker_equals_oracle():
    dev = require_gpu()
    rows = mx_every_amax_rows()
    rows = rows[((rows & 0x7FFF) < 0x7F80).all(axis=1)]
    w = dev_bf16(rows, dev)
    q_t, e_t = torch_mx8(w)
    q_o, e_o = oracle.mx8_quantize(rows)
    assert np.array_equal(host(q_t), q_o) and np.array_equal(host(e_t), e_o)
    w = workloads.kaiming_uniform((512, 2048), seed=4, device=dev)
    q_t, e_t = torch_mx8(w)
    q_o, e_o = oracle.mx8_quantize(workloads.bits(w).reshape(512, 2048))
    assert np.array_equal(host(q_t), q_o) and np.array_equal(host(e_t), e_o)


# ------------------------------------------------------- full-size outputs --

@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2])
def test_pi05_quantize_every_block(fmt):
    """All 27,343,750 blocks of the 3.5e9-element gradient."""
    dev = require_gpu()
    n = workloads.PI05_N
    x = workloads.segmented_gradient(n, seed=0, device=dev)
    q, s = fq.fp8q_quantize(x, fmt)
    torch.cuda.synchronize()
    bad_q = bad_s = 0
    for a in range(0, n, CHUNK):
        b = min(n, a + CHUNK)
        q_t, s_t = torch_quantize(x[a:b], fmt)
        bad_q += _mismatch(q[a:b], q_t)
        bad_s += _mismatch(s[a // 128:b // 128].view(torch.int32), s_t.view(torch.int32))
    assert bad_q == 0 and bad_s == 0, (bad_q, bad_s)


def test_pi05_reduce_every_element():
    """k = 8 peers x 437,500,000 elements (96-element tail) into fp32 and bf16."""
    dev = require_gpu()
    n, k = workloads.PI05_SHARD_N, workloads.PI05_PEERS
    shards = [workloads.random_wire_shard(n, seed=200 + p, fmt=fq.E4M3, device=dev) for p in range(k)]
    qs = [a for a, _ in shards]
    ss = [b for _, b in shards]
    y = fq.fp8q_dequant_reduce(qs, ss, fq.E4M3)
    yb = fq.fp8q_dequant_reduce(qs, ss, fq.E4M3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    bad = bad_b = 0
    for a in range(0, n, CHUNK):
        b = min(n, a + CHUNK)
        ref = torch_reduce(qs, ss, fq.E4M3, a, b)
        bad += _mismatch(y[a:b].view(torch.int32), ref.view(torch.int32))
        bad_b += _mismatch(yb[a:b].view(torch.int16), ref.to(torch.bfloat16).view(torch.int16))
    assert bad == 0 and bad_b == 0, (bad, bad_b)


def test_moe_layer_mx8_every_row():
    """Every row of the 128-expert gate, up and down tensors."""
    dev = require_gpu()
    for name, w in workloads.moe_layer(seed=0, device=dev).items():
        q, e = fq.mx8_quantize(w)
        torch.cuda.synchronize()
        K = w.shape[-1]
        w2 = w.view(-1, K)
        q2, e2 = q.view(-1, K), e.view(w2.shape[0], -1)
        step = CHUNK // K
        bad = 0
        for r in range(0, w2.shape[0], step):
            q_t, e_t = torch_mx8(w2[r:r + step])
            bad += _mismatch(q2[r:r + step], q_t) + _mismatch(e2[r:r + step], e_t)
        assert bad == 0, (name, bad)
        del q, e
