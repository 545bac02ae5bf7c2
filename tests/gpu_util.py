"""Helpers for the GPU parity tests: moving bf16 bit patterns and codes
between numpy (the oracle's side) and torch device tensors (the HIP side)."""
import numpy as np
import pytest
import torch

import dequantize_reduce_transfer_amd as fq


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    # On a GPU machine the library must be there: fail loudly, never skip.
    fq.lib()
    return torch.device("cuda:0")


def dev_bf16(bits: np.ndarray, device) -> torch.Tensor:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).to(device).view(torch.bfloat16)


def dev_u8(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def dev_f32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got).ravel()
    want = np.asarray(want).ravel()
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%s: %d mismatches, first at %s: got %s want %s" % (
        what, bad.size, bad[:5].tolist(), got[bad[:5]].tolist(), want[bad[:5]].tolist())


def assert_reduce_parity(got: np.ndarray, want: np.ndarray, mag: np.ndarray, what: str,
                         rel: float = 1e-6):
    """The gate: |gpu - oracle| <= rel * sum_p |d_p| elementwise (NaN where the
    oracle has NaN).  The goal, also asserted: the same bits, since both sides
    take the same operations in the same order."""
    got = np.asarray(got, dtype=np.float32).ravel()
    want = np.asarray(want, dtype=np.float32).ravel()
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_g, nan_w), what + ": NaN positions differ"
    ok = ~nan_w
    g, w = got[ok].astype(np.float64), want[ok].astype(np.float64)
    m = np.asarray(mag, dtype=np.float64).ravel()[ok]
    inf = np.isinf(w)
    assert np.array_equal(g[inf], w[inf]), what + ": infinities differ"
    err = np.abs(g[~inf] - w[~inf])
    lim = rel * m[~inf]
    bad = np.nonzero(err > lim)[0]
    assert bad.size == 0, "%s: %d outside 1e-6 gate" % (what, bad.size)
    assert_bytes_equal(f32_bits(got[ok]), f32_bits(want[ok]), what + " (bitwise)")


def assert_bf16_parity(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got, dtype=np.uint16).ravel()
    want = np.asarray(want, dtype=np.uint16).ravel()
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_w = (want & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_g, nan_w), what + ": NaN positions differ"
    assert_bytes_equal(got[~nan_w], want[~nan_w], what)
