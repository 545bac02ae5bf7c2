"""Seeded synthetic inputs for the FP8 wire codec.

This module only draws random numbers and shapes them into the workloads the
codec is measured and tested on; it holds none of the codec's arithmetic (no
amax, scale, FP8 rounding or reduction).  The same tensors feed both the HIP
library and, in the tests, the CPU oracle.

Every generator works on any torch device.  The small ones draw with numpy
(PCG64) on the host so that their bytes do not depend on the device; the large
ones draw with a seeded ``torch.Generator`` on the target device.

Workloads (the shapes come from the pages):
  * tiny gradient -- 1,048,576 bf16 values, N(0, 1e-3) with 1% outliers x100
    and one all-zero 128-element block;
  * Pi0.5-scale gradient -- the ~7 GB bf16 gradient of a 3.5B-parameter model
    ("How to Speed Up VLA Training Step by Step: A 3x Acceleration Case Study
    on Pi0.5", the PCIe gradient-communication section), drawn N(0, sigma_s)
    per 25M-element segment with sigma_s log-uniform in [1e-6, 1e-2], and the
    8 data-parallel peers' shards of 437.5M elements (a ring all-reduce moving
    12.25 GB per GPU for 7 GB of gradients means 8 ranks);
  * payload sweep -- 64 KiB .. 64 MiB bf16 payloads, N(0, 1) x 1e-3, with the
    767 KiB AllGather crossover and the 64 MiB all-to-all size of "FP8
    Transmission Optimization for VLA Training", "Threshold Changes" bullet;
  * MoE layer -- one Qwen3-30B-A3B-shaped layer (128 experts, gate/up
    [768, 2048], down [2048, 768]), Kaiming-uniform; the model named in
    "perf: Reduce MXFP8 refit weight-transfer overheads", section "Results";
  * stress shards -- 8 peers x 64 MiB bf16 with per-block mixtures of
    heavy-tailed, near-saturation, FP8-subnormal, bf16-subnormal and zero
    blocks.
"""
from __future__ import annotations

import math

import numpy as np
import torch

BLOCK = 128

TINY_N = 1 << 20
TINY_ZERO_BLOCK = 4096                       # elements [524288, 524416) are zero

PI05_N = 3_500_000_000
PI05_SEGMENT = 25_000_000
PI05_PEERS = 8
PI05_SHARD_N = PI05_N // PI05_PEERS          # 437,500,000 (ends in a 96-element block)

SWEEP_BYTES = (65536, 262144, 785408, 4194304, 16777216, 67108864)

MOE_EXPERTS = 128
MOE_HIDDEN = 2048
MOE_INTER = 768

STRESS_N = 33_554_432                        # 64 MiB of bf16 per peer
STRESS_PEERS = 8
STRESS_CHUNKS = 8                            # all-to-all chunks, one per GPU

E4M3 = 0
E5M2 = 1
_FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}      # only for placing near-max stress values


def _bf16(x: torch.Tensor) -> torch.Tensor:
    """float32 -> bfloat16 by torch's cast (round to nearest even)."""
    return x.to(torch.bfloat16)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def bits(t: torch.Tensor) -> np.ndarray:
    """A bf16 tensor's bit patterns as a host uint16 array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()


# --------------------------------------------------------------------------- #
# tiny gradient                                                               #
# --------------------------------------------------------------------------- #

def tiny_gradient(seed: int = 0, n: int = TINY_N, device="cpu",
                  zero_block: int | None = TINY_ZERO_BLOCK) -> torch.Tensor:
    """N(0, 1e-3), 1% of entries multiplied by 100, one all-zero block."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)
    mask = rng.random(n) < 0.01
    x[mask] *= np.float32(100.0)
    if zero_block is not None and (zero_block + 1) * BLOCK <= n:
        x[zero_block * BLOCK:(zero_block + 1) * BLOCK] = 0.0
    return _bf16(torch.from_numpy(x)).to(device)


# --------------------------------------------------------------------------- #
# Pi0.5-scale gradient                                                         #
# --------------------------------------------------------------------------- #

def segmented_gradient(n: int, seed: int, device="cpu", segment: int = PI05_SEGMENT,
                       std_lo: float = 1e-6, std_hi: float = 1e-2,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """N(0, sigma_s) per segment of ``segment`` elements, sigma_s log-uniform
    in [std_lo, std_hi] (geometric centre 1e-4)."""
    g = _gen(seed, device)
    nseg = max(1, math.ceil(n / segment))
    lo, hi = math.log10(std_lo), math.log10(std_hi)
    sig = torch.pow(10.0, lo + (hi - lo) * torch.rand(nseg, generator=g, device=device,
                                                      dtype=torch.float64))
    sig = sig.cpu().tolist()
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for s in range(nseg):
        a, b = s * segment, min(n, (s + 1) * segment)
        z = torch.randn(b - a, generator=g, device=device, dtype=torch.float32)
        z.mul_(sig[s])
        out[a:b].copy_(z)                       # cast to bf16, RNE
        del z
    return out


def pi05_peer_shard(peer: int, n: int = PI05_SHARD_N, device="cpu") -> torch.Tensor:
    """Peer p's gradient shard: the segmented generator with seed p."""
    return segmented_gradient(n, seed=peer, device=device)


# --------------------------------------------------------------------------- #
# payload sweep                                                                #
# --------------------------------------------------------------------------- #

def sweep_payload(nbytes: int, seed: int, device="cpu") -> torch.Tensor:
    """N(0, 1) x 1e-3 bf16 payload of ``nbytes`` bytes."""
    n = nbytes // 2
    g = _gen(seed, device)
    z = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    return _bf16(z.mul_(1e-3))


# --------------------------------------------------------------------------- #
# MoE layer weights                                                            #
# --------------------------------------------------------------------------- #

def kaiming_uniform(shape, seed: int, device="cpu") -> torch.Tensor:
    """U(-b, b) with b = sqrt(6 / fan_in), fan_in = the last dimension (K)."""
    g = _gen(seed, device)
    b = math.sqrt(6.0 / shape[-1])
    u = torch.rand(*shape, generator=g, device=device, dtype=torch.float32)
    return _bf16(u.mul_(2.0 * b).sub_(b))


def moe_layer(seed: int = 0, experts: int = MOE_EXPERTS, hidden: int = MOE_HIDDEN,
              inter: int = MOE_INTER, device="cpu") -> dict:
    """{'gate': [E, inter, hidden], 'up': [E, inter, hidden], 'down': [E, hidden, inter]}."""
    return {
        "gate": kaiming_uniform((experts, inter, hidden), seed * 3 + 0, device),
        "up": kaiming_uniform((experts, inter, hidden), seed * 3 + 1, device),
        "down": kaiming_uniform((experts, hidden, inter), seed * 3 + 2, device),
    }


# --------------------------------------------------------------------------- #
# stress payload                                                               #
# --------------------------------------------------------------------------- #

STRESS_MIX = (("student_t", 0.70), ("near_max", 0.10), ("fp8_subnormal", 0.08),
              ("bf16_subnormal", 0.04), ("zero", 0.08))


def stress_payload(seed: int, fmt: int, n: int = STRESS_N, device="cpu") -> torch.Tensor:
    """Per 128-element block, one of: Student-t(nu=2) x 1e-3; magnitudes in
    [0.75 M, M] (M = the format's largest finite value); one element +-1e-3
    with the rest at 1e-3 x 2^-U (U in [14, 20] for e4m3, [29, 34] for e5m2),
    so that quotients sweep the FP8 subnormal range and the rounding-to-zero
    threshold; bf16-subnormal magnitudes; all-zero blocks (half of them -0).
    No inf or NaN.  ``n`` must be a multiple of 128."""
    if n % BLOCK:
        raise ValueError("stress payloads are whole blocks")
    g = _gen(seed, device)
    nb = n // BLOCK
    f32 = torch.float32
    u_cat = torch.rand(nb, generator=g, device=device, dtype=f32)
    edges = np.cumsum([w for _, w in STRESS_MIX])
    cat = torch.bucketize(u_cat, torch.tensor(edges[:-1], dtype=f32, device=device), right=True)
    cat = cat.repeat_interleave(BLOCK)
    sign = torch.where(torch.rand(n, generator=g, device=device, dtype=f32) < 0.5, -1.0, 1.0)

    # heavy tailed: t = z / sqrt(chi2_2 / 2), chi2_2 = -2 ln U
    z = torch.randn(n, generator=g, device=device, dtype=f32)
    uu = torch.rand(n, generator=g, device=device, dtype=f32).clamp_min_(1e-30)
    t = z / torch.sqrt(-torch.log(uu)) * 1e-3

    m = _FMT_MAX[fmt]
    near = sign * (0.75 * m + 0.25 * m * torch.rand(n, generator=g, device=device, dtype=f32))

    lo, hi = (14.0, 20.0) if fmt == E4M3 else (29.0, 34.0)
    e = lo + (hi - lo) * torch.rand(n, generator=g, device=device, dtype=f32)
    sub = sign * 1e-3 * torch.pow(2.0, -e)
    lead = torch.zeros(n, dtype=torch.bool, device=device)
    lead[::BLOCK] = True
    sub = torch.where(lead, sign * 1e-3, sub)

    out = _bf16(torch.where(cat == 0, t, torch.where(cat == 1, near, sub)))
    ob = out.view(torch.int16)

    # bf16 subnormals: exponent field 0, mantissa 1..127, random sign
    mant = torch.randint(1, 128, (n,), generator=g, device=device, dtype=torch.int32)
    sbit = (sign < 0).to(torch.int32) << 15
    subn = (mant | sbit).to(torch.int16)
    ob = torch.where(cat == 3, subn, ob)

    # zero blocks, half of them -0
    neg_block = (torch.rand(nb, generator=g, device=device, dtype=f32) < 0.5).repeat_interleave(BLOCK)
    zero = torch.where(neg_block, torch.tensor(-32768, dtype=torch.int16, device=device),
                       torch.tensor(0, dtype=torch.int16, device=device))
    ob = torch.where(cat == 4, zero, ob)
    return ob.view(torch.bfloat16)


# --------------------------------------------------------------------------- #
# synthetic wire shards (codes and scales drawn directly)                      #
# --------------------------------------------------------------------------- #

def random_wire_shard(n: int, seed: int, fmt: int, device="cpu",
                      std_lo: float = 1e-6, std_hi: float = 1e-2):
    """FP8 codes (every finite, non-NaN code equally likely) and positive fp32
    per-block scales log-uniform in [std_lo / 448, std_hi]: a stand-in for a
    peer's wire chunk when only the receiver side is under test."""
    g = _gen(seed, device)
    nb = (n + BLOCK - 1) // BLOCK
    raw = torch.randint(0, 256, (n,), generator=g, device=device, dtype=torch.int32)
    if fmt == E4M3:
        bad = (raw & 0x7F) == 0x7F
        raw = torch.where(bad, raw ^ 0x01, raw)                 # 0x7F -> 0x7E
    else:
        bad = (raw & 0x7F) >= 0x7C
        raw = torch.where(bad, raw - 4, raw)                    # 0x7C.. -> 0x78..
    q = raw.to(torch.uint8)
    lo, hi = math.log10(std_lo / 448.0), math.log10(std_hi)
    s = torch.pow(10.0, lo + (hi - lo) * torch.rand(nb, generator=g, device=device,
                                                    dtype=torch.float64)).to(torch.float32)
    return q, s
