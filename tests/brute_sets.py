"""Deterministic brute-force input sets (bf16 bit patterns), shared by the
oracle and the HIP path in the parity tests.  Construction only: no amax,
scale or rounding happens here.

  B1  every one of the 65536 bf16 patterns alone in a block of zeros, at a
      position that cycles through all 128 lanes of a block;
  B2  all 65536 patterns in natural bit order (512 blocks);
  B3  anchor sweeps: for each of the 128 bf16 significands A in [1, 2) at a
      few binades (ordinary, below 2^-60 where the kernel rescales, and near
      the 2^-126 scale floor), blocks holding A and every finite bf16 whose
      magnitude is at most A (both signs), 127 of them per block, with A's
      position cycling through the block.  By power-of-two invariance this
      spans every (significand ratio, exponent gap) the quantizer can meet.
"""
from __future__ import annotations

from functools import lru_cache

import numpy as np

BLOCK = 128


def b1_single_value_blocks() -> np.ndarray:
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = np.zeros((65536, BLOCK), np.uint16)
    x[np.arange(65536), np.arange(65536) % BLOCK] = v
    return x.ravel()


def b2_natural_order() -> np.ndarray:
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


@lru_cache(maxsize=None)
def _finite_magnitudes() -> np.ndarray:
    m = np.arange(0x7F80, dtype=np.uint32).astype(np.uint16)     # +0 .. max finite
    return m


def b3_anchor_sweep(anchor_exponents=(127, 57, 8)) -> np.ndarray:
    """anchor_exponents are bf16 exponent fields: 127 -> A in [1, 2),
    57 -> A in [2^-70, 2^-69), 8 -> A in [2^-119, 2^-118)."""
    mags = _finite_magnitudes()
    out = []
    nblk = 0
    for e in anchor_exponents:
        for m in range(128):
            a = np.uint16((e << 7) | m)
            small = mags[mags <= a]
            vals = np.concatenate([small, small | np.uint16(0x8000)])
            nb = (vals.size + 126) // 127
            pad = np.zeros(nb * 127, np.uint16)
            pad[:vals.size] = vals
            body = pad.reshape(nb, 127)
            blocks = np.empty((nb, BLOCK), np.uint16)
            pos = (np.arange(nb) + nblk) % BLOCK
            for i in range(nb):
                p = pos[i]
                blocks[i, :p] = body[i, :p]
                blocks[i, p] = a if (i % 2 == 0) else (a | np.uint16(0x8000))
                blocks[i, p + 1:] = body[i, p:]
            nblk += nb
            out.append(blocks.ravel())
    return np.concatenate(out)


def mx_every_amax_rows() -> np.ndarray:
    """[65536, 32]: row r holds bf16 pattern r at column r % 32, zeros elsewhere."""
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = np.zeros((65536, 32), np.uint16)
    w[np.arange(65536), np.arange(65536) % 32] = v
    return w
