"""Exact-rational, brute-force FP8 rounding used to pin the oracle's converter.

This is deliberately a *different computation* from the oracle's encoder:
  * the set of representable values comes from PyTorch's own FP8 dtypes
    (``torch.float8_e4m3fn`` / ``torch.float8_e5m2`` reinterpreting each of
    the 256 codes), not from a decode formula;
  * rounding is a search for the nearest representable value in exact
    rational arithmetic (``fractions.Fraction``), ties going to the code with
    an even last bit, and anything beyond the largest finite value mapping to
    that value (saturation), with the sign carried separately.
"""
from __future__ import annotations

import bisect
import math
from fractions import Fraction
from functools import lru_cache

import numpy as np
import torch

_TORCH_FP8 = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


@lru_cache(maxsize=None)
def code_table(fmt: int):
    """All 256 codes decoded by torch, as float32 numpy values."""
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(_TORCH_FP8[fmt]).to(torch.float32).numpy()


@lru_cache(maxsize=None)
def _positive_grid(fmt: int):
    """Sorted finite non-negative values with their codes (0x00 for zero)."""
    vals = code_table(fmt)
    pairs = {}
    for c in range(128):                      # sign bit clear
        v = float(vals[c])
        if math.isfinite(v):
            pairs.setdefault(Fraction(v), c)   # +0 only once
    grid = sorted(pairs.items())
    return [g[0] for g in grid], [g[1] for g in grid]


def nearest_code(y: float, fmt: int) -> int:
    """Round the real value y (a Python float, exact) to FP8 by brute force."""
    if math.isnan(y):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0x00
    vals, codes = _positive_grid(fmt)
    if math.isinf(y):
        return sign | codes[-1]
    a = Fraction(abs(y))
    if a >= vals[-1]:
        return sign | codes[-1]
    j = bisect.bisect_left(vals, a)
    if vals[j] == a:
        return sign | codes[j]
    lo, hi = j - 1, j
    dlo, dhi = a - vals[lo], vals[hi] - a
    if dlo < dhi:
        pick = lo
    elif dhi < dlo:
        pick = hi
    else:                                      # tie: the even code wins
        pick = lo if codes[lo] % 2 == 0 else hi
    return sign | codes[pick]


def nearest_codes(values: np.ndarray, fmt: int) -> np.ndarray:
    return np.array([nearest_code(float(v), fmt) for v in np.asarray(values).ravel()],
                    dtype=np.uint8).reshape(np.shape(values))
