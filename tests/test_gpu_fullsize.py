"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the same entry points on the same sizes).  Where the oracle
cannot redo the whole output in seconds, sampled blocks / elements are
checked exactly: every block (and every reduced element) depends only on its
own inputs, so a sample is checked by running the oracle on just those
inputs."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
import oracle
from dequantize_reduce_transfer_amd import workloads
from gpu_util import (assert_bf16_parity, assert_bytes_equal, assert_reduce_parity, f32_bits,
                      host, require_gpu)
from helpers import torch_fp8_decode

pytestmark = pytest.mark.gpu


def _sample(nunits, count, seed, always=()):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(min(64, nunits)), np.arange(max(0, nunits - 64), nunits),
                          rng.integers(0, nunits, count), np.asarray(always, dtype=np.int64)])
    return np.unique(idx[(idx >= 0) & (idx < nunits)])


def test_pi05_gradient_quantize_e4m3_full():
    """3.5e9-element bf16 gradient (~7 GB), one launch."""
    dev = require_gpu()
    n = workloads.PI05_N
    x = workloads.segmented_gradient(n, seed=0, device=dev)
    q, s = fq.fp8q_quantize(x, fq.E4M3)
    torch.cuda.synchronize()
    nb = n // 128
    seg_edges = [(k * workloads.PI05_SEGMENT) // 128 for k in range(1, n // workloads.PI05_SEGMENT)]
    idx = _sample(nb, 8192, seed=1, always=seg_edges)
    it = torch.from_numpy(idx).to(dev)
    xb = host(x.view(-1, 128)[it])
    qb = host(q.view(-1, 128)[it])
    sb = host(s[it])
    q_o, s_o = oracle.quantize(xb.ravel(), fq.E4M3)
    assert_bytes_equal(qb.ravel(), q_o, "pi05 sampled codes")
    assert_bytes_equal(f32_bits(sb), f32_bits(s_o), "pi05 sampled scales")


def test_pi05_reduce_k8_full():
    """8 peer shards of 437,500,000 elements (3,417,969 blocks, 96-element tail) -> fp32."""
    dev = require_gpu()
    n, k = workloads.PI05_SHARD_N, workloads.PI05_PEERS
    shards = [workloads.random_wire_shard(n, seed=200 + p, fmt=fq.E4M3, device=dev) for p in range(k)]
    qs = [a for a, _ in shards]
    ss = [b for _, b in shards]
    y = fq.fp8q_dequant_reduce(qs, ss, fq.E4M3)
    torch.cuda.synchronize()
    idx = _sample(n, 16384, seed=2, always=np.arange(n - 300, n))
    it = torch.from_numpy(idx).to(dev)
    bt = torch.from_numpy(idx // 128).to(dev)
    m = idx.size
    # each sampled element becomes element 0 of its own 128-block
    q_in, s_in = [], []
    for q, s in zip(qs, ss):
        qq = np.zeros((m, 128), np.uint8)
        qq[:, 0] = host(q[it])
        q_in.append(qq.ravel())
        s_in.append(host(s[bt]))
    want = oracle.dequant_reduce(q_in, s_in, fq.E4M3)[::128]
    got = host(y[it])
    mag = np.zeros(m)
    for qq, s in zip(q_in, s_in):
        mag += np.abs(torch_fp8_decode(qq[::128], fq.E4M3).astype(np.float64) * s)
    assert_reduce_parity(got, want, mag, "pi05 reduce sampled")


@pytest.mark.parametrize("name", ["gate", "up", "down"])
def test_moe_layer_mx8_full(name):
    """One Qwen3-30B-A3B-shaped MoE layer: 128 experts."""
    dev = require_gpu()
    experts, hidden, inter = workloads.MOE_EXPERTS, workloads.MOE_HIDDEN, workloads.MOE_INTER
    shape = (experts, inter, hidden) if name != "down" else (experts, hidden, inter)
    seed = {"gate": 0, "up": 1, "down": 2}[name]
    w = workloads.kaiming_uniform(shape, seed, device=dev)
    q, e = fq.mx8_quantize(w)
    torch.cuda.synchronize()
    K = shape[-1]
    rows = w.numel() // K
    assert tuple(e.shape) == (rows, K // 32)
    idx = _sample(rows, 512, seed=3 + seed)
    it = torch.from_numpy(idx).to(dev)
    wr = host(w.view(rows, K)[it])
    q_o, e_o = oracle.mx8_quantize(wr)
    assert_bytes_equal(host(q.view(rows, K)[it]), q_o, name + " codes")
    assert_bytes_equal(host(e[it]), e_o, name + " e8m0")


@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2])
def test_stress_full_payload_bf16(fmt):
    """8 peers x 33,554,432 elements (64 MiB bf16 each), reduced into bf16."""
    dev = require_gpu()
    n = workloads.STRESS_N
    bits = [workloads.bits(workloads.stress_payload(p, fmt, n=n, device=dev)) for p in range(8)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        shards = list(ex.map(lambda b: oracle.quantize(b, fmt), bits))
    del bits
    qs = [torch.from_numpy(a).to(dev) for a, _ in shards]
    ss = [torch.from_numpy(b).to(dev) for _, b in shards]
    y = fq.fp8q_dequant_reduce(qs, ss, fmt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.dequant_reduce([a for a, _ in shards], [b for _, b in shards], fmt, out_bf16=True)
    assert_bf16_parity(host(y), want, "stress full")


def test_quantize_and_reduce_beyond_2_pow_32_elements():
    """n = 2^32 + 12345: element offsets past 32 bits, a ragged last block."""
    dev = require_gpu()
    n = (1 << 32) + 12345
    x = workloads.segmented_gradient(n, seed=3, device=dev, segment=1 << 28)
    q, s = fq.fp8q_quantize(x, fq.E4M3)
    torch.cuda.synchronize()
    nb = (n + 127) // 128
    idx = _sample(nb - 1, 4096, seed=4, always=[(1 << 32) // 128 - 1, (1 << 32) // 128,
                                                (1 << 32) // 128 + 1])
    it = torch.from_numpy(idx).to(dev)
    xb = host(x[:(nb - 1) * 128].view(-1, 128)[it])
    q_o, s_o = oracle.quantize(xb.ravel(), fq.E4M3)
    assert_bytes_equal(host(q[:(nb - 1) * 128].view(-1, 128)[it]).ravel(), q_o, "codes")
    assert_bytes_equal(f32_bits(host(s[it])), f32_bits(s_o), "scales")
    tail_x = workloads.bits(x[(nb - 1) * 128:])
    tq, ts = oracle.quantize(tail_x, fq.E4M3)
    assert_bytes_equal(host(q[(nb - 1) * 128:]), tq, "tail codes")
    assert_bytes_equal(f32_bits(host(s[nb - 1:])), f32_bits(ts), "tail scale")
    del x
    # the same codes as two peers of a reduce into bf16 (past 2^32 elements)
    y = fq.fp8q_dequant_reduce([q, q], [s, s], fq.E4M3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    eidx = np.unique(np.concatenate([np.random.default_rng(6).integers(0, n, 8192),
                                     np.arange(n - 300, n), (1 << 32) + np.arange(-64, 64)]))
    et = torch.from_numpy(eidx).to(dev)
    bt = torch.from_numpy(eidx // 128).to(dev)
    m = eidx.size
    qq = np.zeros((m, 128), np.uint8)
    qq[:, 0] = host(q[et])
    sv = host(s[bt])
    want = oracle.dequant_reduce([qq.ravel()] * 2, [sv] * 2, fq.E4M3, out_bf16=True)[::128]
    assert_bf16_parity(host(y[et]), want, "reduce past 2^32")


def test_requantize_beyond_2_pow_32_elements():
    """The reduce -> requantize of one shard of n = 2^32 + 12345 elements
    (e4m3 in, e5m2 out): blocks around element 2^32, the ragged last block
    and random blocks against the oracle."""
    dev = require_gpu()
    n = (1 << 32) + 12345
    x = workloads.segmented_gradient(n, seed=5, device=dev, segment=1 << 28)
    q, s = fq.fp8q_quantize(x, fq.E4M3)
    del x
    q2, s2 = fq.fp8q_dequant_reduce_requantize([q], [s], fq.E4M3, fq.E5M2)
    torch.cuda.synchronize()
    nb = (n + 127) // 128
    idx = _sample(nb - 1, 4096, seed=8, always=[(1 << 32) // 128 - 1, (1 << 32) // 128,
                                                (1 << 32) // 128 + 1])
    it = torch.from_numpy(idx).to(dev)
    qb = host(q[:(nb - 1) * 128].view(-1, 128)[it]).ravel()
    q_o, s_o = oracle.reduce_requantize([qb], [host(s[it])], fq.E4M3, fq.E5M2)
    assert_bytes_equal(host(q2[:(nb - 1) * 128].view(-1, 128)[it]).ravel(), q_o, "codes")
    assert_bytes_equal(f32_bits(host(s2[it])), f32_bits(s_o), "scales")
    tq, ts = oracle.reduce_requantize([host(q[(nb - 1) * 128:])], [host(s[nb - 1:])], fq.E4M3,
                                      fq.E5M2)
    assert_bytes_equal(host(q2[(nb - 1) * 128:]), tq, "tail codes")
    assert_bytes_equal(f32_bits(host(s2[nb - 1:])), f32_bits(ts), "tail scale")
    del q, s, q2, s2
    torch.cuda.empty_cache()


def test_mx8_quantize_and_dequantize_beyond_2_pow_32_elements():
    """MXFP8 of a [2^21 + 1, 2048] weight (2^32 + 2048 elements; the last row
    starts at element 2^32) and its receiver's dequantize into bf16: rows
    around element 2^32 and random rows against the oracle."""
    dev = require_gpu()
    rows, K = (1 << 21) + 1, 2048
    w = workloads.kaiming_uniform((rows, K), seed=9, device=dev)
    q, e = fq.mx8_quantize(w)
    torch.cuda.synchronize()
    idx = _sample(rows, 512, seed=10, always=[(1 << 21) - 2, (1 << 21) - 1, 1 << 21])
    it = torch.from_numpy(idx).to(dev)
    q_o, e_o = oracle.mx8_quantize(host(w[it]))
    assert_bytes_equal(host(q[it]), q_o, "mx codes")
    assert_bytes_equal(host(e[it]), e_o, "mx e8m0")
    del w
    y = fq.mx8_dequantize(q, e, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16_parity(host(y[it]), oracle.mx8_dequantize(q_o, e_o, out_bf16=True), "mx dequantize")
    del q, e, y
    torch.cuda.empty_cache()


def test_pi05_gradient_quantize_e5m2_full():
    """The same 3.5e9-element gradient quantized to e5m2 (sampled blocks)."""
    dev = require_gpu()
    n = workloads.PI05_N
    x = workloads.segmented_gradient(n, seed=0, device=dev)
    q, s = fq.fp8q_quantize(x, fq.E5M2)
    torch.cuda.synchronize()
    idx = _sample(n // 128, 8192, seed=11)
    it = torch.from_numpy(idx).to(dev)
    q_o, s_o = oracle.quantize(host(x.view(-1, 128)[it]).ravel(), fq.E5M2)
    assert_bytes_equal(host(q.view(-1, 128)[it]).ravel(), q_o, "e5m2 sampled codes")
    assert_bytes_equal(f32_bits(host(s[it])), f32_bits(s_o), "e5m2 sampled scales")


# ---------------------------------------------------------------------------
# The same full-size outputs checked in full by the oracle itself, streamed:
# block-aligned chunks are copied to the host and the oracle runs on them
# from a pool of host threads (its C calls release the GIL).  Every block and
# every reduced element depends only on its own inputs, so a chunked oracle
# run equals one run over the whole tensor.

def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _pieces(a, b, parts, multiple):
    step = max(multiple, -(-(-(-(b - a) // parts)) // multiple) * multiple)
    return [(i, min(b, i + step)) for i in range(a, b, step)]


@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2])
def test_pi05_gradient_quantize_every_block_by_the_oracle(fmt):
    """All 27,343,750 blocks of the 3.5e9-element gradient against the oracle."""
    dev = require_gpu()
    n = workloads.PI05_N
    x = workloads.segmented_gradient(n, seed=0, device=dev)
    q, s = fq.fp8q_quantize(x, fmt)
    torch.cuda.synchronize()
    batch = 1 << 28
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        for a in range(0, n, batch):
            b = min(n, a + batch)
            xb = workloads.bits(x[a:b])
            qb, sb = host(q[a:b]), host(s[a // 128:(b + 127) // 128])
            parts = _pieces(0, b - a, 4 * _threads(), 128)
            outs = list(ex.map(lambda p: oracle.quantize(xb[p[0]:p[1]], fmt), parts))
            for (i, j), (q_o, s_o) in zip(parts, outs):
                assert_bytes_equal(qb[i:j], q_o, "codes [%d, %d)" % (a + i, a + j))
                assert_bytes_equal(f32_bits(sb[i // 128:(j + 127) // 128]), f32_bits(s_o),
                                   "scales [%d, %d)" % (a + i, a + j))


def test_pi05_peer_shard_quantize_tail_and_canaries_by_the_oracle():
    """One 437,500,000-element peer shard (a 96-element last block) written
    into larger buffers: every code and scale against the oracle, and the
    canaries past the end untouched."""
    dev = require_gpu()
    n = workloads.PI05_SHARD_N
    x = workloads.pi05_peer_shard(3, n, device=dev)
    nb = fq.num_scales(n)
    qbuf = torch.full((n + 4096,), 0x5A, dtype=torch.uint8, device=dev)
    sbuf = torch.full((nb + 64,), -7.0, dtype=torch.float32, device=dev)
    fq.fp8q_quantize(x, fq.E4M3, q_out=qbuf[:n], scales_out=sbuf[:nb])
    torch.cuda.synchronize()
    xb = workloads.bits(x)
    parts = _pieces(0, n, 4 * _threads(), 128)
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        outs = list(ex.map(lambda p: oracle.quantize(xb[p[0]:p[1]], fq.E4M3), parts))
    qh, sh = host(qbuf), host(sbuf)
    assert_bytes_equal(qh[:n], np.concatenate([o[0] for o in outs]), "codes")
    assert_bytes_equal(f32_bits(sh[:nb]), f32_bits(np.concatenate([o[1] for o in outs])), "scales")
    assert np.all(qh[n:] == 0x5A) and np.all(sh[nb:] == -7.0)


def test_pi05_reduce_k8_every_element_by_the_oracle():
    """All 437,500,000 outputs of the k = 8 reduce (fp32 and bf16) against the oracle."""
    dev = require_gpu()
    n, k = workloads.PI05_SHARD_N, workloads.PI05_PEERS
    shards = [workloads.random_wire_shard(n, seed=200 + p, fmt=fq.E4M3, device=dev) for p in range(k)]
    qs = [a for a, _ in shards]
    ss = [b for _, b in shards]
    y = fq.fp8q_dequant_reduce(qs, ss, fq.E4M3)
    yb = fq.fp8q_dequant_reduce(qs, ss, fq.E4M3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    batch = 1 << 26
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        for a in range(0, n, batch):
            b = min(n, a + batch)
            qh = [host(q[a:b]) for q in qs]
            sh = [host(s[a // 128:(b + 127) // 128]) for s in ss]
            yh, ybh = host(y[a:b]), host(yb[a:b])
            parts = _pieces(0, b - a, 4 * _threads(), 128)

            def run(p, bf):
                i, j = p
                return oracle.dequant_reduce([v[i:j] for v in qh],
                                             [v[i // 128:(j + 127) // 128] for v in sh],
                                             fq.E4M3, out_bf16=bf)
            want = np.concatenate(list(ex.map(lambda p: run(p, False), parts)))
            want_b = np.concatenate(list(ex.map(lambda p: run(p, True), parts)))
            assert_bytes_equal(f32_bits(yh), f32_bits(want), "fp32 [%d, %d)" % (a, b))
            assert_bf16_parity(ybh, want_b, "bf16 [%d, %d)" % (a, b))


def test_moe_layer_mx8_every_row_by_the_oracle():
    """Every row of the 128-expert gate, up and down tensors against the oracle."""
    dev = require_gpu()
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        for name, w in workloads.moe_layer(seed=0, device=dev).items():
            q, e = fq.mx8_quantize(w)
            torch.cuda.synchronize()
            K = w.shape[-1]
            rows = w.numel() // K
            wb = workloads.bits(w).reshape(rows, K)
            parts = _pieces(0, rows, 4 * _threads(), 1)
            outs = list(ex.map(lambda p: oracle.mx8_quantize(wb[p[0]:p[1]]), parts))
            assert_bytes_equal(host(q).reshape(rows, K), np.concatenate([o[0] for o in outs]),
                               name + " codes")
            assert_bytes_equal(host(e), np.concatenate([o[1] for o in outs]), name + " e8m0")
