"""Small test-side helpers: bf16 <-> fp32 through PyTorch's own conversions."""
from __future__ import annotations

import numpy as np
import torch


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), rounded by torch (RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit patterns -> exact fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()


def all_bf16_patterns() -> np.ndarray:
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def finite_bf16_patterns() -> np.ndarray:
    b = all_bf16_patterns()
    return b[(b & 0x7F80) != 0x7F80]


def torch_fp8_decode(codes, fmt: int) -> np.ndarray:
    """Decode FP8 codes with torch's FP8 dtypes (a library routine)."""
    dt = torch.float8_e4m3fn if fmt == 0 else torch.float8_e5m2
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(dt).to(torch.float32).numpy()


def same_bits_f32(a, b) -> bool:
    """Bitwise equality of fp32 arrays, every NaN counted equal to every NaN."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    if a.shape != b.shape:
        return False
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def same_bits_bf16(a, b) -> bool:
    """Bitwise equality of bf16 bit-pattern arrays, NaN payloads not compared."""
    a = np.asarray(a, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    if a.shape != b.shape:
        return False
    na = (a & 0x7FFF) > 0x7F80
    nb = (b & 0x7FFF) > 0x7F80
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a[~na], b[~nb])
