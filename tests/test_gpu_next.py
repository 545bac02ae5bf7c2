"""GPU parity for the next rows, through the C ABI, against the oracle:
dequant-reduce -> requantize, the MXFP8 receiver side (dequantize and k-peer
reduce) and tensorwise quantize.  Codes and scales bit-exact; reductions
bit-exact (which implies the 1e-6 gate)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
import oracle
from dequantize_reduce_transfer_amd import workloads
from gpu_util import (assert_bf16_parity, assert_bytes_equal, dev_bf16, dev_f32, dev_u8, f32_bits,
                      host, require_gpu)

pytestmark = pytest.mark.gpu
FMTS = [fq.E4M3, fq.E5M2]


def _nan_aware_f32(got, want, what):
    got, want = np.asarray(got, np.float32), np.asarray(want, np.float32)
    assert np.array_equal(np.isnan(got), np.isnan(want)), what + ": NaN positions"
    ok = ~np.isnan(want)
    assert_bytes_equal(f32_bits(got[ok]), f32_bits(want[ok]), what)


# --------------------------------------------------------------------------- #
# dequant-reduce -> requantize                                                 #
# --------------------------------------------------------------------------- #

def _check_requant(qs, ss, fin, fout, dev, what):
    q, s = fq.fp8q_dequant_reduce_requantize([dev_u8(a, dev) for a in qs],
                                             [dev_f32(b, dev) for b in ss], fin, fout)
    torch.cuda.synchronize()
    q_o, s_o = oracle.reduce_requantize(qs, ss, fin, fout)
    assert_bytes_equal(host(q), q_o, what + " codes")
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), what + " scales")


@pytest.mark.parametrize("fin,fout", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_requantize_tiny_k4(fin, fout):
    dev = require_gpu()
    shards = [oracle.quantize(workloads.bits(workloads.tiny_gradient(p)), fin) for p in range(4)]
    _check_requant([a for a, _ in shards], [b for _, b in shards], fin, fout, dev, "tiny k=4")


@pytest.mark.parametrize("k", list(range(1, 17)))
def test_requantize_every_peer_count(k):
    dev = require_gpu()
    n = 128 * 200 + 51
    shards = [workloads.random_wire_shard(n, seed=500 + 17 * k + p, fmt=1) for p in range(k)]
    _check_requant([a.numpy() for a, _ in shards], [b.numpy() for _, b in shards], 1, 0, dev,
                   "k=%d" % k)


@pytest.mark.parametrize("n", [1, 100, 128, 129, 511, 512, 513, 1023, 1024, 1025, 3000])
def test_requantize_ragged_leaves_canaries(n):
    dev = require_gpu()
    k = 8
    shards = [workloads.random_wire_shard(n, seed=n + p, fmt=0) for p in range(k)]
    qs = [dev_u8(a.numpy(), dev) for a, _ in shards]
    ss = [dev_f32(b.numpy(), dev) for _, b in shards]
    nb = (n + 127) // 128
    q_big = torch.full((n + 64,), 0x33, dtype=torch.uint8, device=dev)
    s_big = torch.full((nb + 8,), 9.0, dtype=torch.float32, device=dev)
    fq.fp8q_dequant_reduce_requantize(qs, ss, 0, 0, q_out=q_big[:n], scales_out=s_big[:nb])
    torch.cuda.synchronize()
    q_o, s_o = oracle.reduce_requantize([a.numpy() for a, _ in shards], [b.numpy() for _, b in shards], 0, 0)
    qh, sh = host(q_big), host(s_big)
    assert_bytes_equal(qh[:n], q_o, "codes")
    assert_bytes_equal(f32_bits(sh[:nb]), f32_bits(s_o), "scales")
    assert np.all(qh[n:] == 0x33) and np.all(sh[nb:] == 9.0)


def test_requantize_nonfinite_and_cancelling_blocks():
    dev = require_gpu()
    n = 128 * 8
    q0 = np.zeros(n, np.uint8)
    q0[5] = 0x7C                      # e5m2 +inf
    q0[300] = 0x7F                    # e5m2 NaN
    q0[600:700] = 0x3C                # 1.0
    q1 = q0.copy()
    q1[600:700] = 0xBC                # -1.0: block 4 and 5 cancel to zeros
    s = np.ones(8, np.float32)
    _check_requant([q0, q1], [s, s], 1, 0, dev, "specials")


@pytest.mark.parametrize("fmt", FMTS)
def test_requantize_stress_share(fmt):
    dev = require_gpu()
    n = workloads.STRESS_N // workloads.STRESS_CHUNKS
    bits = [workloads.bits(workloads.stress_payload(p, fmt, n=n)) for p in range(8)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        shards = list(ex.map(lambda b: oracle.quantize(b, fmt), bits))
    _check_requant([a for a, _ in shards], [b for _, b in shards], fmt, fmt, dev, "stress share")


# --------------------------------------------------------------------------- #
# MXFP8 receiver side                                                          #
# --------------------------------------------------------------------------- #

def test_mx8_dequantize_every_code_with_scale_samples():
    dev = require_gpu()
    q = np.tile(np.arange(256, dtype=np.uint8), 64).reshape(64, 256)
    e = (np.arange(64 * 8, dtype=np.int64) * 37 % 256).astype(np.uint8).reshape(64, 8)
    e[0, :] = [0, 1, 2, 127, 128, 253, 254, 255]
    for dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        y = host(fq.mx8_dequantize(dev_u8(q, dev), dev_u8(e, dev), out_dtype=dt))
        want = oracle.mx8_dequantize(q, e, out_bf16=bf)
        if bf:
            assert_bf16_parity(y.ravel(), want.ravel(), "every code bf16")
        else:
            _nan_aware_f32(y.ravel(), want.ravel(), "every code f32")


@pytest.mark.parametrize("name", ["gate", "up", "down"])
def test_mx8_roundtrip_moe_shapes(name):
    dev = require_gpu()
    layer = workloads.moe_layer(seed=1, experts=4)
    w = workloads.bits(layer[name]).reshape(layer[name].shape)
    q, e = oracle.mx8_quantize(w)
    y = host(fq.mx8_dequantize(dev_u8(q, dev), dev_u8(e, dev)))
    _nan_aware_f32(y.ravel(), oracle.mx8_dequantize(q.reshape(-1, q.shape[-1]), e).ravel(), name)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 8, 11, 16])
def test_mx8_reduce_every_peer_count(k):
    dev = require_gpu()
    rows, K = 37, 320
    shards = [oracle.mx8_quantize(workloads.bits(workloads.kaiming_uniform((rows, K), seed=700 + p))
                                  .reshape(rows, K)) for p in range(k)]
    qd = [dev_u8(a, dev) for a, _ in shards]
    ed = [dev_u8(b, dev) for _, b in shards]
    for dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        y = host(fq.mx8_dequant_reduce(qd, ed, out_dtype=dt))
        want = oracle.mx8_dequant_reduce([a for a, _ in shards], [b for _, b in shards], out_bf16=bf)
        if bf:
            assert_bf16_parity(y.ravel(), want.ravel(), "k=%d bf16" % k)
        else:
            _nan_aware_f32(y.ravel(), want.ravel(), "k=%d f32" % k)


MXR_SWITCH = [(1023, 2048, 4), (1024, 2048, 4), (1023, 2048, 8), (1024, 2048, 3)]


@pytest.mark.parametrize("rows,K,k", MXR_SWITCH, ids=["r%d-K%d-k%d" % c for c in MXR_SWITCH])
def test_mx8_reduce_small_launch_switch(rows, K, k):
    """From 4 peers, below 2^21 elements the MXFP8 receiver takes one tile
    of one group per wave: [1023, 2048] and [1024, 2048] shards (and 3
    peers, which keep the deeper tile), fp32 and bf16, against the oracle."""
    dev = require_gpu()
    shards = [oracle.mx8_quantize(workloads.bits(workloads.kaiming_uniform((rows, K), seed=720 + p))
                                  .reshape(rows, K)) for p in range(k)]
    qd = [dev_u8(a, dev) for a, _ in shards]
    ed = [dev_u8(b, dev) for _, b in shards]
    for dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        y = host(fq.mx8_dequant_reduce(qd, ed, out_dtype=dt))
        want = oracle.mx8_dequant_reduce([a for a, _ in shards], [b for _, b in shards], out_bf16=bf)
        if bf:
            assert_bf16_parity(y.ravel(), want.ravel(), "rows=%d k=%d bf16" % (rows, k))
        else:
            _nan_aware_f32(y.ravel(), want.ravel(), "rows=%d k=%d f32" % (rows, k))


@pytest.mark.parametrize("rows,K", [(255, 2048), (256, 2048), (1365, 768), (4099, 160)])
def test_mx8_dequantize_bf16_every_byte(rows, K):
    """The MXFP8 dequantize into bf16 at [255, 2048], [256, 2048] (2^19
    elements) and ragged [1365, 768] and [4099, 160]: every code byte and
    E8M0 byte drawn (NaN codes, the NaN scale 0xFF and the scale floor 0x00
    included), canaries after the output, every bf16 against the oracle."""
    dev = require_gpu()
    rng = np.random.default_rng(rows + K)
    q = rng.integers(0, 256, (rows, K)).astype(np.uint8)
    e = rng.integers(0, 256, (rows, K // 32)).astype(np.uint8)
    n = rows * K
    y_big = torch.full((n + 40,), -2.5, dtype=torch.bfloat16, device=dev)
    fq.mx8_dequantize(dev_u8(q, dev), dev_u8(e, dev), out_dtype=torch.bfloat16,
                      out=y_big[:n].view(rows, K))
    torch.cuda.synchronize()
    yh = host(y_big)
    assert_bf16_parity(yh[:n], oracle.mx8_dequantize(q, e, out_bf16=True).ravel(),
                       "mx dequantize bf16 %dx%d" % (rows, K))
    assert np.all(yh[n:] == 0xC020)


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 96), (9, 256), (64, 2048), (129, 768)])
def test_mx8_dequantize_ragged_leaves_canaries(rows, K):
    dev = require_gpu()
    rng = np.random.default_rng(rows * K)
    q = rng.integers(0, 256, (rows, K)).astype(np.uint8)
    e = rng.integers(0, 256, (rows, K // 32)).astype(np.uint8)
    n = rows * K
    y_big = torch.full((n + 40,), -2.5, dtype=torch.float32, device=dev)
    fq.mx8_dequantize(dev_u8(q, dev), dev_u8(e, dev), out=y_big[:n].view(rows, K))
    torch.cuda.synchronize()
    yh = host(y_big)
    _nan_aware_f32(yh[:n], oracle.mx8_dequantize(q, e).ravel(), "ragged")
    assert np.all(yh[n:] == -2.5)


# --------------------------------------------------------------------------- #
# tensorwise                                                                   #
# --------------------------------------------------------------------------- #

def _check_tensorwise(bits, fmt, dev, what):
    q, s = fq.fp8q_quantize_tensorwise(dev_bf16(bits, dev), fmt)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_tensorwise(bits, fmt)
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), what + " scale")
    assert_bytes_equal(host(q), q_o, what + " codes")


@pytest.mark.parametrize("fmt", FMTS)
def test_tensorwise_tiny(fmt):
    dev = require_gpu()
    _check_tensorwise(workloads.bits(workloads.tiny_gradient(0)), fmt, dev, "tiny")


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 127, 128, 2047, 2048, 2049, 65536 + 5, 1 << 22])
def test_tensorwise_ragged_sizes(n):
    dev = require_gpu()
    rng = np.random.default_rng(n)
    f = (rng.standard_normal(n) * np.exp(rng.uniform(-10, 10, n))).astype(np.float32)
    bits = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x = dev_bf16(bits, dev)
    q_big = torch.full((n + 64,), 0x5C, dtype=torch.uint8, device=dev)
    s_big = torch.full((4,), 5.0, dtype=torch.float32, device=dev)
    fq.fp8q_quantize_tensorwise(x, 1, q_out=q_big[:n], scale_out=s_big[:1])
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_tensorwise(bits, 1)
    qh, sh = host(q_big), host(s_big)
    assert_bytes_equal(qh[:n], q_o, "codes")
    assert_bytes_equal(f32_bits(sh[:1]), f32_bits(s_o), "scale")
    assert np.all(qh[n:] == 0x5C) and np.all(sh[1:] == 5.0)


def test_tensorwise_zero_tiny_and_nonfinite():
    dev = require_gpu()
    for bits in (np.zeros(5000, np.uint16),
                 np.full(3000, 0x8001, np.uint16),                       # bf16 subnormals
                 np.concatenate([np.full(4000, 0x3F80, np.uint16), [0x7F80]]).astype(np.uint16)):
        for fmt in FMTS:
            _check_tensorwise(bits, fmt, dev, "special")


def test_tensorwise_repeated_calls_reset_the_amax():
    """The scale slot carries the amax only during a call: a second call on a
    smaller tensor must not see the first call's larger amax."""
    dev = require_gpu()
    xt = workloads.tiny_gradient(1)
    big = workloads.bits(xt)
    small = workloads.bits((xt[:4096].float() * 2.0 ** -6).to(torch.bfloat16))   # 64x smaller
    s = torch.empty(1, dtype=torch.float32, device=dev)
    q1 = torch.empty(big.size, dtype=torch.uint8, device=dev)
    q2 = torch.empty(small.size, dtype=torch.uint8, device=dev)
    fq.fp8q_quantize_tensorwise(dev_bf16(big, dev), 0, q_out=q1, scale_out=s)
    fq.fp8q_quantize_tensorwise(dev_bf16(small, dev), 0, q_out=q2, scale_out=s)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_tensorwise(small, 0)
    assert_bytes_equal(host(q2), q_o, "second call codes")
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), "second call scale")


def test_tensorwise_pi05_gradient_full_sampled():
    """3.5e9 elements: sampled codes checked by the oracle on the sample plus
    the tensor's largest element (found by torch), which has the same amax."""
    dev = require_gpu()
    n = workloads.PI05_N
    x = workloads.segmented_gradient(n, seed=0, device=dev)
    q, s = fq.fp8q_quantize_tensorwise(x, fq.E4M3)
    torch.cuda.synchronize()
    imax = int(torch.argmax(x.view(torch.int16).bitwise_and(0x7FFF)).item())
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([rng.integers(0, n, 200_000), np.arange(1000),
                                    np.arange(n - 1000, n), [imax]]))
    it = torch.from_numpy(idx).to(dev)
    xs = workloads.bits(x[it])
    q_o, s_o = oracle.quantize_tensorwise(xs, fq.E4M3)
    assert_bytes_equal(f32_bits(host(s)), f32_bits(s_o), "scale")
    assert_bytes_equal(host(q[it]), q_o, "sampled codes")


@pytest.mark.parametrize("fmt_out", [fq.E4M3, fq.E5M2])
def test_requantize_quotient_across_every_scale_range(fmt_out):
    """Sums whose blocks span fp32 from subnormal to 2^100: block scales set
    to 2^e * (1 + m) for every exponent e in [-149, 100], so amax falls below
    2^-60 (the rescaled quotient), near the 2^-126 scale floor and far above,
    with every code present; compared with the oracle byte for byte."""
    dev = require_gpu()
    rng = np.random.default_rng(17)
    exps = np.arange(-149, 101)
    nb = exps.size * 4
    n = nb * 128
    qs, ss = [], []
    for p in range(2):
        q = rng.integers(0, 256, n).astype(np.uint8)
        q[(q & 0x7F) == 0x7F] ^= 0x01                   # no NaN codes (e4m3 input)
        sig = 1.0 + rng.random(nb)
        s = np.ldexp(sig, np.repeat(exps, 4)).astype(np.float32)
        s[s == 0] = np.float32(2.0 ** -149)
        qs.append(q)
        ss.append(s)
    q_g, s_g = fq.fp8q_dequant_reduce_requantize([dev_u8(a, dev) for a in qs],
                                                 [dev_f32(b, dev) for b in ss], fq.E4M3, fmt_out)
    torch.cuda.synchronize()
    q_o, s_o = oracle.reduce_requantize(qs, ss, fq.E4M3, fmt_out)
    assert_bytes_equal(host(q_g), q_o, "codes")
    assert_bytes_equal(f32_bits(host(s_g)), f32_bits(s_o), "scales")


RQ_SWITCH = [((1 << 22) - 1, 2), (1 << 22, 2), ((1 << 22) + 77, 3), ((1 << 24) - 1, 8),
             (1 << 24, 8), ((1 << 24) - 1, 16)]


@pytest.mark.parametrize("n,k", RQ_SWITCH, ids=["n%d-k%d" % c for c in RQ_SWITCH])
def test_requantize_shape_switch_sizes(n, k):
    """Below 2^22 elements (2^24 from 4 peers) the requantize takes one tile
    of one 512-element group per wave; above, two tiles of two (ending in
    one-tile waves from 4 peers): one element either side of each switch,
    e4m3 -> e5m2, every code and scale against the oracle."""
    dev = require_gpu()
    shards = [workloads.random_wire_shard(n, seed=950 + 10 * k + p, fmt=0) for p in range(k)]
    _check_requant([a.numpy() for a, _ in shards], [b.numpy() for _, b in shards], 0, 1, dev,
                   "switch n=%d k=%d" % (n, k))


@pytest.mark.parametrize("k", [4, 8, 16])
def test_requantize_one_tile_tail_sizes(k):
    """From 4 peers and 2^23 elements the requantize ends with one-tile waves
    (its last 4096 tiles): a ragged size past that, e5m2 -> e4m3, every code
    and scale against the oracle.  Special blocks are planted at the start
    and among the one-tile waves: an inf and a NaN code, peers that cancel
    to a zero block, sums below 2^-60 (tiny scales), and sums that overflow
    fp32 to inf (huge scales)."""
    dev = require_gpu()
    n = (1 << 23) + 1024 * 321 + 77
    shards = [workloads.random_wire_shard(n, seed=900 + 10 * k + p, fmt=1) for p in range(k)]
    qs = [a.numpy().copy() for a, _ in shards]
    ss = [b.numpy().copy() for _, b in shards]
    for base in (0, (n - 1024 * 1000) // 128 * 128, (n - 2048 - 77) // 128 * 128):
        b0 = base // 128
        qs[0][base + 5] = 0x7C                          # +inf
        qs[1][base + 128 + 9] = 0x7F                    # NaN
        for p in range(k):                              # block b0 + 2 cancels: +1, -1, +1, -1 ...
            qs[p][base + 256:base + 384] = 0x3C if p % 2 == 0 else 0xBC
            ss[p][b0 + 2] = 1.0
        for p in range(k):                              # block b0 + 3: sums near 2^-100
            ss[p][b0 + 3] = 2.0 ** -110
        for p in range(k):                              # block b0 + 4: 57344 * 2^115 overflows
            qs[p][base + 512:base + 640] = 0x7B
            ss[p][b0 + 4] = 2.0 ** 115
    _check_requant(qs, ss, 1, 0, dev, "tail k=%d" % k)
