"""CPU oracle for the FP8 wire codec -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never calls it, and the two share no code:
the arithmetic lives in ``fp8q_oracle.c`` (plain C, built with gcc) and this
module only marshals numpy arrays into it with ctypes.

Each function cites the passage of the pages it follows in the C source.
Formats: ``E4M3`` / ``E5M2`` are the OCP FP8 formats (OFP8 rev 1.0).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

E4M3 = 0
E5M2 = 1
BLOCK = 128
MX_BLOCK = 32

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8q_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile fp8q_oracle.c into liboracle.so with gcc (no GPU involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # The mutation test points this at a deliberately broken build.
    path = os.environ.get("FP8Q_ORACLE_LIB", _LIB_PATH)
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    S = ctypes.c_size_t
    I = ctypes.c_int
    lib.oracle_fp8_encode.argtypes = [ctypes.c_double, I]
    lib.oracle_fp8_encode.restype = ctypes.c_uint8
    lib.oracle_fp8_decode.argtypes = [ctypes.c_uint8, I]
    lib.oracle_fp8_decode.restype = ctypes.c_float
    lib.oracle_fp8_max.argtypes = [I]
    lib.oracle_fp8_max.restype = ctypes.c_double
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_fp8_encode_f32_array.argtypes = [P, S, I, P]
    lib.oracle_fp8_decode_array.argtypes = [P, S, I, P]
    lib.oracle_quantize.argtypes = [P, S, I, P, P]
    lib.oracle_dequantize.argtypes = [P, P, S, I, P, I]
    lib.oracle_dequant_reduce.argtypes = [P, P, I, S, I, P, I]
    lib.oracle_mx8_quantize.argtypes = [P, S, S, P, P]
    lib.oracle_mx8_quantize.restype = I
    lib.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_decode.restype = ctypes.c_float
    lib.oracle_quantize_tensorwise.argtypes = [P, S, I, P, P]
    lib.oracle_reduce_requantize.argtypes = [P, P, I, S, I, I, P, P]
    lib.oracle_mx8_dequant_reduce.argtypes = [P, P, I, S, S, P, I]
    lib.oracle_mx8_dequant_reduce.restype = I
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def fp8_max(fmt: int) -> float:
    return _load().oracle_fp8_max(fmt)


def fp8_encode(y, fmt: int) -> np.ndarray:
    """satRNE of fp32 values to FP8 codes (uint8)."""
    y = _c(np.asarray(y, dtype=np.float32), np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    _load().oracle_fp8_encode_f32_array(_ptr(y), y.size, fmt, _ptr(out))
    return out


def fp8_encode_exact(v: float, fmt: int) -> int:
    """satRNE of one real value given as a Python float (a double)."""
    return int(_load().oracle_fp8_encode(float(v), fmt))


def fp8_decode(codes, fmt: int) -> np.ndarray:
    c = _c(np.asarray(codes, dtype=np.uint8), np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    _load().oracle_fp8_decode_array(_ptr(c), c.size, fmt, _ptr(out))
    return out


def e8m0_decode(code: int) -> float:
    return float(_load().oracle_e8m0_decode(code))


def f32_to_bf16(v: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(v)))


def num_blocks(n: int, block: int = BLOCK) -> int:
    return (n + block - 1) // block


def quantize(x_bits, fmt: int):
    """Block-128 quantize of bf16 bit patterns -> (q uint8[n], scales f32[ceil(n/128)])."""
    x = _c(x_bits, np.uint16).reshape(-1)
    n = x.size
    q = np.empty(n, dtype=np.uint8)
    s = np.empty(num_blocks(n), dtype=np.float32)
    if n:
        _load().oracle_quantize(_ptr(x), n, fmt, _ptr(q), _ptr(s))
    return q, s


def dequantize(q, scales, fmt: int, out_bf16: bool = False) -> np.ndarray:
    q = _c(q, np.uint8).reshape(-1)
    s = _c(scales, np.float32).reshape(-1)
    n = q.size
    if s.size < num_blocks(n):
        raise ValueError("too few scales")
    y = np.empty(n, dtype=np.uint16 if out_bf16 else np.float32)
    if n:
        _load().oracle_dequantize(_ptr(q), _ptr(s), n, fmt, _ptr(y), int(out_bf16))
    return y


def dequant_reduce(qs, ss, fmt: int, out_bf16: bool = False) -> np.ndarray:
    k = len(qs)
    if k < 1 or k != len(ss):
        raise ValueError("need k >= 1 shards with one scale array each")
    qs = [_c(q, np.uint8).reshape(-1) for q in qs]
    ss = [_c(s, np.float32).reshape(-1) for s in ss]
    n = qs[0].size
    for q, s in zip(qs, ss):
        if q.size != n or s.size < num_blocks(n):
            raise ValueError("shard shape mismatch")
    qp = (ctypes.c_void_p * k)(*[_ptr(q) for q in qs])
    sp = (ctypes.c_void_p * k)(*[_ptr(s) for s in ss])
    y = np.empty(n, dtype=np.uint16 if out_bf16 else np.float32)
    if n:
        _load().oracle_dequant_reduce(qp, sp, k, n, fmt, _ptr(y), int(out_bf16))
    return y


def mx8_quantize(w_bits):
    """MXFP8 quantize of bf16 weights [..., K] -> (q uint8 same shape, e8m0 uint8 [rows, K/32])."""
    w = _c(w_bits, np.uint16)
    if w.ndim < 1:
        raise ValueError("need at least one dimension")
    K = w.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    rows = w.size // K if K else 0
    q = np.empty(w.shape, dtype=np.uint8)
    e = np.empty((rows, K // MX_BLOCK), dtype=np.uint8)
    if w.size:
        rc = _load().oracle_mx8_quantize(_ptr(w), rows, K, _ptr(q), _ptr(e))
        if rc != 0:
            raise ValueError("oracle rejected K")
    return q, e


def quantize_tensorwise(x_bits, fmt: int):
    """One fp32 scale for the whole tensor -> (q uint8[n], scale f32[1])."""
    x = _c(x_bits, np.uint16).reshape(-1)
    q = np.empty(x.size, dtype=np.uint8)
    s = np.empty(1, dtype=np.float32)
    if x.size == 0:
        s[0] = 2.0 ** -126
        return q, s
    _load().oracle_quantize_tensorwise(_ptr(x), x.size, fmt, _ptr(q), _ptr(s))
    return q, s


def reduce_requantize(qs, ss, fmt_in: int, fmt_out: int):
    """Dequant-reduce k shards, then block-128 quantize the fp32 sums."""
    k = len(qs)
    if k < 1 or k != len(ss):
        raise ValueError("need k >= 1 shards with one scale array each")
    qs = [_c(q, np.uint8).reshape(-1) for q in qs]
    ss = [_c(s, np.float32).reshape(-1) for s in ss]
    n = qs[0].size
    for q, s in zip(qs, ss):
        if q.size != n or s.size < num_blocks(n):
            raise ValueError("shard shape mismatch")
    qp = (ctypes.c_void_p * k)(*[_ptr(q) for q in qs])
    sp = (ctypes.c_void_p * k)(*[_ptr(s) for s in ss])
    q_out = np.empty(n, dtype=np.uint8)
    s_out = np.empty(num_blocks(n), dtype=np.float32)
    if n:
        _load().oracle_reduce_requantize(qp, sp, k, n, fmt_in, fmt_out, _ptr(q_out), _ptr(s_out))
    return q_out, s_out


def mx8_dequant_reduce(qs, es, out_bf16: bool = False) -> np.ndarray:
    """Ordered fp32 sum over k MXFP8 shards (q [rows, K], e8m0 [rows, K/32])."""
    k = len(qs)
    if k < 1 or k != len(es):
        raise ValueError("need k >= 1 shards with one scale array each")
    qs = [_c(q, np.uint8) for q in qs]
    es = [_c(e, np.uint8) for e in es]
    K = qs[0].shape[-1]
    rows = qs[0].size // K if K else 0
    for q, e in zip(qs, es):
        if q.shape != qs[0].shape or e.size != rows * (K // MX_BLOCK):
            raise ValueError("shard shape mismatch")
    qp = (ctypes.c_void_p * k)(*[_ptr(q) for q in qs])
    ep = (ctypes.c_void_p * k)(*[_ptr(e) for e in es])
    y = np.empty(qs[0].shape, dtype=np.uint16 if out_bf16 else np.float32)
    if qs[0].size:
        if _load().oracle_mx8_dequant_reduce(qp, ep, k, rows, K, _ptr(y), int(out_bf16)) != 0:
            raise ValueError("K must be a multiple of 32")
    return y


def mx8_dequantize(q, e8m0, out_bf16: bool = False) -> np.ndarray:
    return mx8_dequant_reduce([q], [e8m0], out_bf16)
