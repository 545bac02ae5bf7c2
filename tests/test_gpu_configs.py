"""Each workload's whole chain on the GPU, on that workload's own inputs.

For every workload that quantizes and then reduces, the peers' shards are
made by the GPU quantize (not by the oracle, and not drawn as wire codes);
every code and scale of every shard is compared with the oracle's quantize of
the same bf16 input; then the GPU reduces its own shards and every output is
compared with the oracle's reduce of the oracle's shards.  The oracle never
takes an input from the HIP path: the two chains only meet in the
comparisons, and the first comparison shows their shards are the same bytes.

  tiny gradient     1,048,576 elements, peers seeds 0-3: quantize,
                    dequantize, k = 4 reduce (e4m3 and e5m2, fp32 and bf16)
  Pi0.5 gradient    8 peers x 437,500,000 elements (96-element last block),
                    e4m3: quantize, k = 8 reduce into fp32 and bf16
  payload sweep     64 KiB .. 64 MiB, 8 peers (seeds 0-7), e5m2: quantize,
                    k = 8 reduce into fp32 and bf16
  stress payload    8 peers x 33,554,432 elements, e4m3 and e5m2: quantize,
                    k = 8 reduce into bf16 of the full payload and of one
                    GPU's share (all-to-all chunk 0)

Large outputs are compared in block-aligned pieces from a pool of host
threads; every block and every reduced element depends only on its own
inputs, so the pieces together equal one whole run of the oracle.
"""
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

FMTS = [fq.E4M3, fq.E5M2]


def _threads():
    """The host's CPU share for one GPU is 16; use at most that many."""
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _pieces(n, parts, multiple=128):
    step = max(multiple, -(-(-(-n // parts)) // multiple) * multiple)
    return [(i, min(n, i + step)) for i in range(0, n, step)]


def _oracle_quantize(ex, xb, fmt):
    """oracle.quantize over block-aligned pieces of one bf16 array."""
    outs = list(ex.map(lambda p: oracle.quantize(xb[p[0]:p[1]], fmt),
                       _pieces(xb.size, 4 * _threads())))
    return np.concatenate([o[0] for o in outs]), np.concatenate([o[1] for o in outs])


def _oracle_reduce(ex, qs, ss, fmt, out_bf16):
    """oracle.dequant_reduce over block-aligned pieces of k shards."""
    n = qs[0].size

    def run(p):
        i, j = p
        return oracle.dequant_reduce([q[i:j] for q in qs], [s[i // 128:(j + 127) // 128] for s in ss],
                                     fmt, out_bf16=out_bf16)
    return np.concatenate(list(ex.map(run, _pieces(n, 4 * _threads()))))


def _magnitudes(qs, ss, fmt):
    """sum_p |d_p| per element, for the 1e-6 relative gate."""
    mag = np.zeros(qs[0].size)
    for q, s in zip(qs, ss):
        mag += np.abs(torch_fp8_decode(q, fmt).astype(np.float64) * np.repeat(s, 128)[:q.size])
    return mag


def _check_shards(ex, xs_bits, qd, sd, fmt, what):
    """Every code and scale of the GPU-made shards against the oracle's
    quantize of the same inputs; returns the oracle's shards."""
    shards = []
    for p, xb in enumerate(xs_bits):
        q_o, s_o = _oracle_quantize(ex, xb, fmt)
        assert_bytes_equal(host(qd[p]), q_o, "%s peer %d codes" % (what, p))
        assert_bytes_equal(f32_bits(host(sd[p])), f32_bits(s_o), "%s peer %d scales" % (what, p))
        shards.append((q_o, s_o))
    return shards


@pytest.mark.parametrize("fmt", FMTS)
def test_tiny_gradient_chain(fmt):
    """Quantize the four seeded tiny gradients, dequantize each, reduce all
    four (k = 4) into fp32 and bf16."""
    dev = require_gpu()
    xs = [workloads.tiny_gradient(p) for p in range(4)]
    bits = [workloads.bits(x) for x in xs]
    qd, sd = zip(*[fq.fp8q_quantize(x.to(dev), fmt) for x in xs])
    deq = [fq.fp8q_dequantize(q, s, fmt) for q, s in zip(qd, sd)]
    deq_bf = [fq.fp8q_dequantize(q, s, fmt, out_dtype=torch.bfloat16) for q, s in zip(qd, sd)]
    y = fq.fp8q_dequant_reduce(list(qd), list(sd), fmt)
    yb = fq.fp8q_dequant_reduce(list(qd), list(sd), fmt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    with ThreadPoolExecutor(_threads()) as ex:
        shards = _check_shards(ex, bits, qd, sd, fmt, "tiny")
    qs = [a for a, _ in shards]
    ss = [b for _, b in shards]
    # the zero block of the workload: all-zero codes, the 2^-126 floor
    z = workloads.TINY_ZERO_BLOCK
    assert np.all(qs[0][z * 128:(z + 1) * 128] == 0) and ss[0][z] == np.float32(2.0 ** -126)
    for p in range(4):
        want = oracle.dequantize(qs[p], ss[p], fmt)
        assert_bytes_equal(f32_bits(host(deq[p])), f32_bits(want), "tiny dequantize %d" % p)
        assert_bf16_parity(host(deq_bf[p]), oracle.dequantize(qs[p], ss[p], fmt, out_bf16=True),
                           "tiny dequantize bf16 %d" % p)
    assert_reduce_parity(host(y), oracle.dequant_reduce(qs, ss, fmt), _magnitudes(qs, ss, fmt),
                         "tiny k=4")
    assert_bf16_parity(host(yb), oracle.dequant_reduce(qs, ss, fmt, out_bf16=True), "tiny k=4 bf16")


@pytest.mark.parametrize("nbytes", workloads.SWEEP_BYTES)
def test_payload_sweep_chain_e5m2(nbytes):
    """Each sweep payload: the 8 seeded peers quantized to e5m2 on the GPU,
    then the k = 8 reduce of those GPU-made shards into fp32 and bf16."""
    dev = require_gpu()
    xs = [workloads.sweep_payload(nbytes, seed=p) for p in range(8)]
    bits = [workloads.bits(x) for x in xs]
    qd, sd = zip(*[fq.fp8q_quantize(x.to(dev), fq.E5M2) for x in xs])
    y = fq.fp8q_dequant_reduce(list(qd), list(sd), fq.E5M2)
    yb = fq.fp8q_dequant_reduce(list(qd), list(sd), fq.E5M2, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    with ThreadPoolExecutor(_threads()) as ex:
        shards = _check_shards(ex, bits, qd, sd, fq.E5M2, "sweep %d B" % nbytes)
        qs = [a for a, _ in shards]
        ss = [b for _, b in shards]
        want = _oracle_reduce(ex, qs, ss, fq.E5M2, False)
        want_b = _oracle_reduce(ex, qs, ss, fq.E5M2, True)
    assert_reduce_parity(host(y), want, _magnitudes(qs, ss, fq.E5M2), "sweep %d B k=8" % nbytes)
    assert_bf16_parity(host(yb), want_b, "sweep %d B k=8 bf16" % nbytes)


@pytest.mark.parametrize("fmt", FMTS)
def test_stress_payload_chain_bf16(fmt):
    """The stress payload's 8 peers quantized on the GPU, then the k = 8
    reduce into bf16 of the full payload and of one GPU's share."""
    dev = require_gpu()
    n, chunks = workloads.STRESS_N, workloads.STRESS_CHUNKS
    xs = [workloads.stress_payload(p, fmt, n=n, device=dev) for p in range(8)]
    qd, sd = zip(*[fq.fp8q_quantize(x, fmt) for x in xs])
    y = fq.fp8q_dequant_reduce(list(qd), list(sd), fmt, out_dtype=torch.bfloat16)
    cn = n // chunks
    ysh = fq.fp8q_dequant_reduce([q[:cn] for q in qd], [s[:cn // 128] for s in sd], fmt,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    bits = [workloads.bits(x) for x in xs]
    del xs
    with ThreadPoolExecutor(_threads()) as ex:
        shards = _check_shards(ex, bits, qd, sd, fmt, "stress")
        qs = [a for a, _ in shards]
        ss = [b for _, b in shards]
        want = _oracle_reduce(ex, qs, ss, fmt, True)
    assert_bf16_parity(host(y), want, "stress full bf16")
    want_sh = oracle.dequant_reduce([q[:cn] for q in qs], [s[:cn // 128] for s in ss], fmt,
                                    out_bf16=True)
    assert_bf16_parity(host(ysh), want_sh, "stress share bf16")


def test_pi05_peer_shards_chain_every_output():
    """The 8 Pi0.5 peers (seed p, 437,500,000 elements, a 96-element last
    block) quantized to e4m3 on the GPU, then the k = 8 reduce of those
    GPU-made shards into fp32 and bf16: every block of every shard and every
    reduced element against the oracle, streamed in block-aligned chunks."""
    dev = require_gpu()
    n, k = workloads.PI05_SHARD_N, workloads.PI05_PEERS
    xs = [workloads.pi05_peer_shard(p, n, device=dev) for p in range(k)]
    qd, sd = zip(*[fq.fp8q_quantize(x, fq.E4M3) for x in xs])
    y = fq.fp8q_dequant_reduce(list(qd), list(sd), fq.E4M3)
    yb = fq.fp8q_dequant_reduce(list(qd), list(sd), fq.E4M3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert n % 128 == 96
    batch = 1 << 26                                 # a multiple of 128
    with ThreadPoolExecutor(_threads()) as ex:
        for a in range(0, n, batch):
            b = min(n, a + batch)
            sa, sb = a // 128, (b + 127) // 128
            qs, ss = [], []
            for p in range(k):
                q_o, s_o = _oracle_quantize(ex, workloads.bits(xs[p][a:b]), fq.E4M3)
                assert_bytes_equal(host(qd[p][a:b]), q_o, "peer %d codes [%d, %d)" % (p, a, b))
                assert_bytes_equal(f32_bits(host(sd[p][sa:sb])), f32_bits(s_o),
                                   "peer %d scales [%d, %d)" % (p, a, b))
                qs.append(q_o)
                ss.append(s_o)
            want = _oracle_reduce(ex, qs, ss, fq.E4M3, False)
            assert_bytes_equal(f32_bits(host(y[a:b])), f32_bits(want), "fp32 [%d, %d)" % (a, b))
            want_b = _oracle_reduce(ex, qs, ss, fq.E4M3, True)
            assert_bf16_parity(host(yb[a:b]), want_b, "bf16 [%d, %d)" % (a, b))
