"""GPU parity: dequantize and fused dequant-reduce (HIP, through the C ABI)
against the oracle.  The reduce's gate is the 1e-6 relative bound on
sum_p |d_p|; since both sides add the same products in the same order, the
bits must match too."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
import oracle
from dequantize_reduce_transfer_amd import workloads
from gpu_util import (assert_bf16_parity, assert_bytes_equal, assert_reduce_parity, dev_f32,
                      dev_u8, f32_bits, host, require_gpu)
from helpers import torch_fp8_decode

pytestmark = pytest.mark.gpu
FMTS = [fq.E4M3, fq.E5M2]


def _magnitudes(qs, ss, fmt):
    """sum_p |dec(q_p) * s_p| in float64, for the relative gate."""
    n = qs[0].size
    m = np.zeros(n, np.float64)
    for q, s in zip(qs, ss):
        d = torch_fp8_decode(q, fmt).astype(np.float64) * np.repeat(s.astype(np.float64), 128)[:n]
        m += np.abs(np.nan_to_num(d, nan=0.0, posinf=0.0, neginf=0.0))
    return m


def _oracle_shards(bits_list, fmt, workers=8):
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda b: oracle.quantize(b, fmt), bits_list))


def _gpu_reduce(qs, ss, fmt, dev, out_dtype=torch.float32):
    qd = [dev_u8(q, dev) for q in qs]
    sd = [dev_f32(s, dev) for s in ss]
    y = fq.fp8q_dequant_reduce(qd, sd, fmt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(y)


def _check_reduce(qs, ss, fmt, dev, what):
    y32 = _gpu_reduce(qs, ss, fmt, dev)
    want32 = oracle.dequant_reduce(qs, ss, fmt)
    assert_reduce_parity(y32, want32, _magnitudes(qs, ss, fmt), what + " f32")
    ybf = _gpu_reduce(qs, ss, fmt, dev, torch.bfloat16)
    assert_bf16_parity(ybf, oracle.dequant_reduce(qs, ss, fmt, out_bf16=True), what + " bf16")


@pytest.mark.parametrize("fmt", FMTS)
def test_tiny_gradient_k4(fmt):
    dev = require_gpu()
    shards = _oracle_shards([workloads.bits(workloads.tiny_gradient(p)) for p in range(4)], fmt)
    qs, ss = [a for a, _ in shards], [b for _, b in shards]
    _check_reduce(qs, ss, fmt, dev, "tiny k=4")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize(fmt, out_dtype):
    dev = require_gpu()
    bits = workloads.bits(workloads.tiny_gradient(2))
    q, s = oracle.quantize(bits, fmt)
    y = fq.fp8q_dequantize(dev_u8(q, dev), dev_f32(s, dev), fmt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    want = oracle.dequantize(q, s, fmt, out_bf16=(out_dtype == torch.bfloat16))
    if out_dtype == torch.float32:
        assert_bytes_equal(f32_bits(host(y)), f32_bits(want), "dequantize f32")
    else:
        assert_bf16_parity(host(y), want, "dequantize bf16")


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_every_code_with_nan_scale(fmt):
    dev = require_gpu()
    q = np.tile(np.arange(256, dtype=np.uint8), 4)
    s = np.array([1.0, 2.0 ** -126, np.nan, 3.0e30, 0.25, 7.0, 1e-20, 65536.0], np.float32)
    y = host(fq.fp8q_dequantize(dev_u8(q, dev), dev_f32(s, dev), fmt))
    want = oracle.dequantize(q, s, fmt)
    assert np.array_equal(np.isnan(y), np.isnan(want))
    ok = ~np.isnan(want)
    assert_bytes_equal(f32_bits(y[ok]), f32_bits(want[ok]), "every code")
    yb = host(fq.fp8q_dequantize(dev_u8(q, dev), dev_f32(s, dev), fmt, out_dtype=torch.bfloat16))
    assert_bf16_parity(yb, oracle.dequantize(q, s, fmt, out_bf16=True), "every code bf16")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", list(range(1, 17)))
def test_every_peer_count(fmt, k):
    dev = require_gpu()
    n = 128 * 300 + 77
    shards = [workloads.random_wire_shard(n, seed=1000 * k + p, fmt=fmt) for p in range(k)]
    qs = [a.numpy() for a, _ in shards]
    ss = [b.numpy() for _, b in shards]
    _check_reduce(qs, ss, fmt, dev, "k=%d" % k)


@pytest.mark.parametrize("n", [1, 5, 127, 128, 255, 256, 257, 1023, 1024, 1025, 4096 + 100])
def test_ragged_sizes_leave_canaries(n):
    dev = require_gpu()
    k = 3
    shards = [workloads.random_wire_shard(n, seed=n + p, fmt=0) for p in range(k)]
    qs = [dev_u8(a.numpy(), dev) for a, _ in shards]
    ss = [dev_f32(b.numpy(), dev) for _, b in shards]
    y_big = torch.full((n + 40,), -3.5, dtype=torch.float32, device=dev)
    fq.fp8q_dequant_reduce(qs, ss, 0, out=y_big[:n])
    yb_big = torch.full((n + 40,), 77, dtype=torch.int16, device=dev)
    fq.fp8q_dequant_reduce(qs, ss, 0, out_dtype=torch.bfloat16, out=yb_big.view(torch.bfloat16)[:n])
    torch.cuda.synchronize()
    qh = [a.numpy() for a, _ in shards]
    sh = [b.numpy() for _, b in shards]
    yh = host(y_big)
    assert_bytes_equal(f32_bits(yh[:n]), f32_bits(oracle.dequant_reduce(qh, sh, 0)), "n=%d" % n)
    assert np.all(yh[n:] == -3.5)
    ybh = host(yb_big)
    assert_bf16_parity(ybh[:n].view(np.uint16), oracle.dequant_reduce(qh, sh, 0, out_bf16=True),
                       "bf16 n=%d" % n)
    assert np.all(ybh[n:] == 77)


@pytest.mark.parametrize("k", [9, 16])
@pytest.mark.parametrize("n", [1, 127, 511, 512, 513, 1025, 4096 + 77])
def test_many_peers_bf16_ragged_sizes_leave_canaries(k, n):
    """From 9 peers up the reduce into bf16 maps eight codes to a lane
    (512-element tiles); around and below one tile only the tail path runs."""
    dev = require_gpu()
    shards = [workloads.random_wire_shard(n, seed=7 * n + p, fmt=1) for p in range(k)]
    qs = [dev_u8(a.numpy(), dev) for a, _ in shards]
    ss = [dev_f32(b.numpy(), dev) for _, b in shards]
    yb_big = torch.full((n + 40,), 77, dtype=torch.int16, device=dev)
    fq.fp8q_dequant_reduce(qs, ss, 1, out_dtype=torch.bfloat16, out=yb_big.view(torch.bfloat16)[:n])
    torch.cuda.synchronize()
    ybh = host(yb_big)
    want = oracle.dequant_reduce([a.numpy() for a, _ in shards], [b.numpy() for _, b in shards], 1,
                                 out_bf16=True)
    assert_bf16_parity(ybh[:n].view(np.uint16), want, "bf16 k=%d n=%d" % (k, n))
    assert np.all(ybh[n:] == 77)


@pytest.mark.parametrize("nbytes", workloads.SWEEP_BYTES)
def test_payload_sweep_e5m2_k8(nbytes):
    dev = require_gpu()
    bits = [workloads.bits(workloads.sweep_payload(nbytes, seed=p)) for p in range(8)]
    shards = _oracle_shards(bits, fq.E5M2)
    qs, ss = [a for a, _ in shards], [b for _, b in shards]
    y = _gpu_reduce(qs, ss, fq.E5M2, dev)
    assert_reduce_parity(y, oracle.dequant_reduce(qs, ss, fq.E5M2),
                         _magnitudes(qs, ss, fq.E5M2), "sweep %d B" % nbytes)


@pytest.mark.parametrize("fmt", FMTS)
def test_stress_share_bf16_out(fmt):
    """One GPU's share of the 64 MiB stress payload: chunk 0 of 8 peers."""
    dev = require_gpu()
    n = workloads.STRESS_N // workloads.STRESS_CHUNKS
    bits = [workloads.bits(workloads.stress_payload(p, fmt, n=n)) for p in range(8)]
    shards = _oracle_shards(bits, fmt)
    qs, ss = [a for a, _ in shards], [b for _, b in shards]
    y = _gpu_reduce(qs, ss, fmt, dev, torch.bfloat16)
    assert_bf16_parity(y, oracle.dequant_reduce(qs, ss, fmt, out_bf16=True), "stress share")


@pytest.mark.parametrize("fmt", FMTS)
def test_naive_path_equals_fused(fmt):
    dev = require_gpu()
    n, k = 128 * 999 + 3, 8
    shards = [workloads.random_wire_shard(n, seed=50 + p, fmt=fmt, device=dev) for p in range(k)]
    qs = [a for a, _ in shards]
    ss = [b for _, b in shards]
    fused = fq.fp8q_dequant_reduce(qs, ss, fmt)
    parts = [fq.fp8q_dequantize(q, s, fmt) for q, s in zip(qs, ss)]
    naive = fq.fp8q_sum_f32(parts)
    naive_bf = fq.fp8q_sum_f32(parts, out_dtype=torch.bfloat16)
    fused_bf = fq.fp8q_dequant_reduce(qs, ss, fmt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int32), naive.view(torch.int32))
    assert torch.equal(fused_bf.view(torch.int16), naive_bf.view(torch.int16))


@pytest.mark.parametrize("fmt", FMTS)
def test_peers_cancel_exactly(fmt):
    dev = require_gpu()
    bits = workloads.bits(workloads.tiny_gradient(4))
    q0, s0 = oracle.quantize(bits, fmt)
    q1, s1 = oracle.quantize(bits ^ 0x8000, fmt)
    y = _gpu_reduce([q0, q1], [s0, s1], fmt, dev)
    assert np.all(y == 0)


def test_same_shard_twice_and_deterministic():
    dev = require_gpu()
    q, s = workloads.random_wire_shard(100_000, seed=9, fmt=0, device=dev)
    a = fq.fp8q_dequant_reduce([q, q, q], [s, s, s], 0)
    b = fq.fp8q_dequant_reduce([q, q, q], [s, s, s], 0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    want = oracle.dequant_reduce([host(q)] * 3, [host(s)] * 3, 0)
    assert_bytes_equal(f32_bits(host(a)), f32_bits(want), "same shard x3")


def test_bf16_output_overflow_rounds_like_rne():
    """fp32 results between bf16's largest finite value and fp32's: RNE sends
    those at or above the midpoint to +-inf and the rest to +-max."""
    dev = require_gpu()
    bf16_max = float(np.array([0x7F7F0000], np.uint32).view(np.float32)[0])
    mid = float(np.array([0x7F7F8000], np.uint32).view(np.float32)[0])
    targets = np.array([bf16_max, np.nextafter(np.float32(mid), np.float32(0)), mid,
                        np.nextafter(np.float32(mid), np.float32(np.inf)), 3.4e38], np.float32)
    n = 128 * targets.size
    q = np.zeros(n, np.uint8)
    q[::128] = 0x38                    # e4m3 1.0: dec * s == s exactly
    q[1::128] = 0xB8                   # -1.0
    s = targets.copy()
    for dt_bf in (False, True):
        y = host(fq.fp8q_dequantize(dev_u8(q, dev), dev_f32(s, dev), 0,
                                    out_dtype=torch.bfloat16 if dt_bf else torch.float32))
        want = oracle.dequantize(q, s, 0, out_bf16=dt_bf)
        if dt_bf:
            assert_bf16_parity(y, want, "bf16 overflow")
            assert (want[::128] == 0x7F80).sum() == 3 and (want[1::128] == 0xFF80).sum() == 3
        else:
            assert_bytes_equal(f32_bits(y), f32_bits(want), "f32")
    # two peers whose fp32 sum overflows
    big = np.full(1, 3.0e38, np.float32)
    qq = np.zeros(128, np.uint8)
    qq[0] = 0x38
    y = host(fq.fp8q_dequant_reduce([dev_u8(qq, dev)] * 2, [dev_f32(big, dev)] * 2, 0))
    assert np.isinf(y[0]) and y[0] > 0


@pytest.mark.parametrize("k", [3, 9, 14])
def test_scales_at_odd_word_offsets(k):
    """Scale arrays only 4-byte aligned (odd word offsets into a larger
    buffer), on the scalar-scale (k = 3, 14) and vector-scale (k = 9) paths,
    for the reduce and the requantize."""
    dev = require_gpu()
    n = 128 * 2000 + 33
    nb = (n + 127) // 128
    shards = [workloads.random_wire_shard(n, seed=500 + p, fmt=fq.E4M3) for p in range(k)]
    qh = [a.numpy() for a, _ in shards]
    sh = [b.numpy() for _, b in shards]
    qd = [dev_u8(a, dev) for a in qh]
    sd = []
    for p, s in enumerate(sh):
        off = 2 * p + 1                                # an odd number of floats
        buf = torch.zeros(nb + off + 3, dtype=torch.float32, device=dev)
        buf[off:off + nb] = torch.from_numpy(s).to(dev)
        sd.append(buf[off:off + nb])
        assert sd[-1].data_ptr() % 8 == 4
    y = fq.fp8q_dequant_reduce(qd, sd, fq.E4M3)
    q_r, s_r = fq.fp8q_dequant_reduce_requantize(qd, sd, fq.E4M3, fq.E5M2)
    torch.cuda.synchronize()
    assert_bytes_equal(f32_bits(host(y)), f32_bits(oracle.dequant_reduce(qh, sh, fq.E4M3)), "reduce")
    q_o, s_o = oracle.reduce_requantize(qh, sh, fq.E4M3, fq.E5M2)
    assert_bytes_equal(host(q_r), q_o, "requantize codes")
    assert_bytes_equal(f32_bits(host(s_r)), f32_bits(s_o), "requantize scales")


@pytest.mark.parametrize("k", [4, 8])
def test_scales_at_odd_word_offsets_mid_size(k):
    """The same at a mid size past 2^23 elements, where the reduce loads its
    scales per lane and ends with one-tile waves (into fp32 and bf16) and the
    requantize ends with one-tile waves too; the requantize's output scales
    also start at an odd word offset, between canaries."""
    dev = require_gpu()
    n = (1 << 23) + 128 * 37 + 5
    nb = (n + 127) // 128
    shards = [workloads.random_wire_shard(n, seed=520 + p, fmt=fq.E5M2) for p in range(k)]
    qh = [a.numpy() for a, _ in shards]
    sh = [b.numpy() for _, b in shards]
    qd = [dev_u8(a, dev) for a in qh]
    sd = []
    for p, s in enumerate(sh):
        off = 2 * p + 3
        buf = torch.zeros(nb + off + 3, dtype=torch.float32, device=dev)
        buf[off:off + nb] = torch.from_numpy(s).to(dev)
        sd.append(buf[off:off + nb])
        assert sd[-1].data_ptr() % 8 == 4
    want = oracle.dequant_reduce(qh, sh, fq.E5M2)
    y = fq.fp8q_dequant_reduce(qd, sd, fq.E5M2)
    yb = fq.fp8q_dequant_reduce(qd, sd, fq.E5M2, out_dtype=torch.bfloat16)
    so_buf = torch.full((nb + 6,), 7.0, dtype=torch.float32, device=dev)
    s_r = so_buf[5:5 + nb]
    assert s_r.data_ptr() % 8 == 4
    q_r, _ = fq.fp8q_dequant_reduce_requantize(qd, sd, fq.E5M2, fq.E4M3, scales_out=s_r)
    torch.cuda.synchronize()
    assert_bytes_equal(f32_bits(host(y)), f32_bits(want), "reduce fp32")
    assert_bf16_parity(host(yb), oracle.dequant_reduce(qh, sh, fq.E5M2, out_bf16=True),
                       "reduce bf16")
    q_o, s_o = oracle.reduce_requantize(qh, sh, fq.E5M2, fq.E4M3)
    assert_bytes_equal(host(q_r), q_o, "requantize codes")
    assert_bytes_equal(f32_bits(host(s_r)), f32_bits(s_o), "requantize scales")
    sb = host(so_buf)
    assert np.all(sb[:5] == 7.0) and np.all(sb[5 + nb:] == 7.0), "requantize scale canaries"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", list(range(2, 9)))
def test_mid_size_every_peer_count(fmt, k):
    """2..8 peers between 2^22 and 2^26 elements take the vector-scale
    loads (each lane fetches its block's scale with the codes): a ragged
    size there, every output against the oracle, fp32 and bf16."""
    dev = require_gpu()
    n = (1 << 22) + 128 * 777 + 45
    shards = [workloads.random_wire_shard(n, seed=5000 + 10 * k + p, fmt=fmt) for p in range(k)]
    qs = [a.numpy() for a, _ in shards]
    ss = [b.numpy() for _, b in shards]
    _check_reduce(qs, ss, fmt, dev, "mid-size k=%d" % k)


SWITCH_CASES = [((1 << 19) - 1, 8, False), (1 << 19, 8, False), (1 << 19, 5, True),
                ((1 << 22) - 1, 8, False), (1 << 22, 8, False), ((1 << 26) - 1, 8, False),
                (1 << 26, 8, False), ((1 << 22) - 1, 5, True), (1 << 22, 5, True),
                ((1 << 22) - 1, 4, True), ((1 << 22) - 1, 1, False), (1 << 22, 1, False),
                ((1 << 22) - 1, 1, True), ((1 << 24) - 1, 12, True), (1 << 24, 12, True),
                ((1 << 24) - 1, 8, False), (1 << 24, 8, False), (1 << 24, 4, False),
                ((1 << 22) - 1, 12, False), (1 << 22, 12, False), ((1 << 27) - 1, 2, False),
                (1 << 27, 2, False), ((1 << 25) - 1, 6, True), (1 << 25, 6, True),
                ((1 << 25) - 1, 3, True), (1 << 25, 3, True),
                ((1 << 19) - 1, 1, True), (1 << 19, 1, True), (1 << 22, 1, True),
                ((11 << 20) - 1, 1, True), (11 << 20, 1, True), (3 * (1 << 25) + 77, 1, True),
                ((1 << 26) - 1, 5, True), (1 << 26, 5, True), ((1 << 27) - 1, 5, True),
                (1 << 27, 5, True)]


@pytest.mark.parametrize("n,k,bf16", SWITCH_CASES,
                         ids=["n%d-k%d-%s" % (c[0], c[1], "bf16" if c[2] else "f32")
                              for c in SWITCH_CASES])
def test_reduce_shape_switch_sizes(n, k, bf16):
    """The launch shape changes at 2^19 elements (from there up to 2^22, one
    tile per wave of one 256-element group into fp32 and into bf16 from 5
    peers), at 2^22 (below it one tile per wave, above it two), at 2^26
    (vector-scale loads end), into bf16 from 9 peers (eight codes per
    lane) at 2^24 (one tile per wave below), and into fp32 at 2^24 (2^22
    from 9 peers) and 2^27, the bounds of the one-group, one-tile band (not
    taken by 4 peers), and into bf16 from 2 peers at 2^25, 2^26 and 2^27,
    where the eight-codes mapping takes over (one tile per wave below 2^26)
    and hands back, and where one shard into bf16 takes it with one tile per
    wave from 2^19, leaves it at 2^22 and takes it again at 11 * 2^20 (with a
    ragged tail at 3 * 2^25 + 77): one element either side of each, every
    output's bits against the oracle."""
    dev = require_gpu()
    shards = [workloads.random_wire_shard(n, seed=6000 + p, fmt=fq.E4M3) for p in range(k)]
    qh = [a.numpy() for a, _ in shards]
    sh = [b.numpy() for _, b in shards]
    out = torch.bfloat16 if bf16 else torch.float32
    y = fq.fp8q_dequant_reduce([dev_u8(a, dev) for a in qh], [dev_f32(b, dev) for b in sh],
                               fq.E4M3, out_dtype=out)
    torch.cuda.synchronize()
    want = oracle.dequant_reduce(qh, sh, fq.E4M3, out_bf16=bf16)
    if bf16:
        assert_bf16_parity(host(y), want, "n=%d k=%d" % (n, k))
    else:
        assert_bytes_equal(f32_bits(host(y)), f32_bits(want), "n=%d k=%d" % (n, k))
