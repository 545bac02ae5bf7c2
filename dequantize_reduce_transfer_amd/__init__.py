"""MI355X-native FP8 wire codec: Python binding of ``libfp8q.so``.

A thin ctypes layer over the C ABI declared in ``include/fp8q.h``: it checks
tensor dtypes and devices, allocates outputs with torch when the caller gives
none, passes raw device pointers and torch's current HIP stream, and turns a
non-zero status into :class:`Fp8qError`.  Every step of the computation runs
in the HIP kernels; there is no CPU fallback, and every call raises if the
library has not been built (``python -m dequantize_reduce_transfer_amd.build``).

Functions (same names as the C entry points):
  fp8q_quantize(x, fmt)                -> (q uint8 [n], scales f32 [ceil(n/128)])
  fp8q_dequantize(q, scales, fmt)      -> y f32 or bf16 [n]
  fp8q_dequant_reduce(qs, ss, fmt)     -> y f32 or bf16 [n]
  mx8_quantize(w)                      -> (q uint8 w.shape, e8m0 uint8 [rows, K/32])
  fp8q_sum_f32(parts)                  -> y f32 or bf16 [n]
  fp8q_dequant_reduce_requantize(qs, ss, fmt_in, fmt_out) -> (q uint8 [n], scales f32)
  mx8_dequantize(q, e8m0)              -> y f32 or bf16, q.shape
  mx8_dequant_reduce(qs, es)           -> y f32 or bf16, q.shape
  fp8q_quantize_tensorwise(x, fmt)     -> (q uint8 [n], scale f32 [1])
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

E4M3 = 0
E5M2 = 1
OUT_F32 = 0
OUT_BF16 = 1
BLOCK = 128
MX_BLOCK = 32
MAX_PEERS = 16

_PKG = os.path.dirname(os.path.abspath(__file__))
# FP8Q_LIB selects another build of the same library (e.g. one compiled with
# a small grid cap to exercise the kernels' grid-stride loops in tests).
LIB_PATH = os.environ.get("FP8Q_LIB") or os.path.join(_PKG, "libfp8q.so")
_lib = None

EXPORTS = ("fp8q_quantize", "fp8q_dequantize", "fp8q_dequant_reduce", "mx8_quantize",
           "fp8q_sum_f32", "fp8q_dequant_reduce_requantize", "mx8_dequantize",
           "mx8_dequant_reduce", "fp8q_quantize_tensorwise", "fp8q_status_str",
           "fp8q_abi_version")


class Fp8qError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded ``libfp8q.so`` with argument types set (raises if unbuilt)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfp8q.so is not built (%s); run "
                           "`python -m dequantize_reduce_transfer_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    PP = ctypes.POINTER(ctypes.c_void_p)
    L.fp8q_quantize.argtypes = [P, S, I, P, P, P]
    L.fp8q_dequantize.argtypes = [P, P, S, I, P, I, P]
    L.fp8q_dequant_reduce.argtypes = [PP, PP, I, S, I, P, I, P]
    L.mx8_quantize.argtypes = [P, S, S, P, P, P]
    L.fp8q_sum_f32.argtypes = [PP, I, S, P, I, P]
    L.fp8q_dequant_reduce_requantize.argtypes = [PP, PP, I, S, I, I, P, P, P]
    L.mx8_dequantize.argtypes = [P, P, S, S, P, I, P]
    L.mx8_dequant_reduce.argtypes = [PP, PP, I, S, S, P, I, P]
    L.fp8q_quantize_tensorwise.argtypes = [P, S, I, P, P, P]
    for f in ("fp8q_quantize", "fp8q_dequantize", "fp8q_dequant_reduce", "mx8_quantize",
              "fp8q_sum_f32", "fp8q_dequant_reduce_requantize", "mx8_dequantize",
              "mx8_dequant_reduce", "fp8q_quantize_tensorwise"):
        getattr(L, f).restype = I
    L.fp8q_status_str.argtypes = [I]
    L.fp8q_status_str.restype = ctypes.c_char_p
    L.fp8q_abi_version.argtypes = []
    L.fp8q_abi_version.restype = I
    _lib = L
    return L


def fp8q_status_str(status: int) -> str:
    return lib().fp8q_status_str(int(status)).decode()


def fp8q_abi_version() -> int:
    return int(lib().fp8q_abi_version())


def _check(status: int, what: str) -> None:
    if status != 0:
        raise Fp8qError(status, "%s: %s" % (what, fp8q_status_str(status)))


def _run(what: str, tensors, fn, *args, stream=None) -> None:
    """Call a C entry point with every tensor on one GPU, that GPU current
    (the library launches on the current HIP device).  When the caller names
    a stream, every tensor is recorded on it, so that torch's caching
    allocator does not hand a tensor's memory to new work while the kernels
    enqueued there may still read or write it."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError("%s: all tensors must be on %s, got one on %s" % (what, dev, t.device))
    if stream is not None and stream.device != dev:
        raise ValueError("%s: the stream is on %s, the tensors on %s" % (what, stream.device, dev))
    with torch.cuda.device(dev):
        _check(fn(*args), what)
    if stream is not None:
        for t in tensors:
            t.record_stream(stream)


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ptrs(ts: Sequence[torch.Tensor]):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _fmt(fmt: int) -> int:
    if fmt not in (E4M3, E5M2):
        raise ValueError("fmt must be E4M3 (0) or E5M2 (1)")
    return fmt


def _out_code(dtype) -> int:
    if dtype == torch.float32:
        return OUT_F32
    if dtype == torch.bfloat16:
        return OUT_BF16
    raise ValueError("output dtype must be torch.float32 or torch.bfloat16")


def num_scales(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


def fp8q_quantize(x: torch.Tensor, fmt: int = E4M3, q_out: Optional[torch.Tensor] = None,
                  scales_out: Optional[torch.Tensor] = None, stream=None):
    """Block-128 quantize of a bf16 tensor (flattened) -> (q, scales)."""
    _need(x, torch.bfloat16, "x")
    n = x.numel()
    if q_out is None:
        q_out = torch.empty(n, dtype=torch.uint8, device=x.device)
    if scales_out is None:
        scales_out = torch.empty(num_scales(n), dtype=torch.float32, device=x.device)
    _need(q_out, torch.uint8, "q_out")
    _need(scales_out, torch.float32, "scales_out")
    if q_out.numel() != n or scales_out.numel() != num_scales(n):
        raise ValueError("q_out must hold n codes and scales_out ceil(n/128) scales")
    _run("fp8q_quantize", [x, q_out, scales_out], lib().fp8q_quantize, x.data_ptr(), n,
         _fmt(fmt), q_out.data_ptr(), scales_out.data_ptr(), _stream(x, stream), stream=stream)
    return q_out, scales_out


def fp8q_dequantize(q: torch.Tensor, scales: torch.Tensor, fmt: int = E4M3,
                    out_dtype=torch.float32, out: Optional[torch.Tensor] = None, stream=None):
    """y = dec(q) * scale per 128-element block, as fp32 or bf16."""
    _need(q, torch.uint8, "q")
    _need(scales, torch.float32, "scales")
    n = q.numel()
    if scales.numel() < num_scales(n):
        raise ValueError("scales must hold ceil(n/128) values")
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=q.device)
    _need(out, out_dtype, "out")
    if out.numel() != n:
        raise ValueError("out must hold n values")
    _run("fp8q_dequantize", [q, scales, out], lib().fp8q_dequantize, q.data_ptr(),
         scales.data_ptr(), n, _fmt(fmt), out.data_ptr(), _out_code(out_dtype), _stream(q, stream), stream=stream)
    return out


def fp8q_dequant_reduce(qs: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
                        fmt: int = E4M3, out_dtype=torch.float32,
                        out: Optional[torch.Tensor] = None, stream=None):
    """Fused sum over k peers of dec(q_p) * s_p, in peer order, fp32 accumulation."""
    k = len(qs)
    if k < 1 or k != len(scales):
        raise ValueError("need k >= 1 code tensors and as many scale tensors")
    if k > MAX_PEERS:
        raise ValueError("at most %d peers" % MAX_PEERS)
    n = qs[0].numel()
    for i, (q, s) in enumerate(zip(qs, scales)):
        _need(q, torch.uint8, "qs[%d]" % i)
        _need(s, torch.float32, "scales[%d]" % i)
        if q.numel() != n or s.numel() < num_scales(n):
            raise ValueError("peer %d has the wrong size" % i)
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=qs[0].device)
    _need(out, out_dtype, "out")
    if out.numel() != n:
        raise ValueError("out must hold n values")
    _run("fp8q_dequant_reduce", [*qs, *scales, out], lib().fp8q_dequant_reduce, _ptrs(qs),
         _ptrs(scales), k, n, _fmt(fmt), out.data_ptr(), _out_code(out_dtype), _stream(qs[0], stream), stream=stream)
    return out


def mx8_quantize(w: torch.Tensor, q_out: Optional[torch.Tensor] = None,
                 e8m0_out: Optional[torch.Tensor] = None, stream=None):
    """MXFP8 quantize of bf16 weights [..., K] -> (q like w, e8m0 [rows, K/32])."""
    _need(w, torch.bfloat16, "w")
    if w.dim() < 1:
        raise ValueError("w needs at least one dimension")
    K = w.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    rows = w.numel() // K if K else 0
    if q_out is None:
        q_out = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if e8m0_out is None:
        e8m0_out = torch.empty((rows, K // MX_BLOCK), dtype=torch.uint8, device=w.device)
    _need(q_out, torch.uint8, "q_out")
    _need(e8m0_out, torch.uint8, "e8m0_out")
    if q_out.numel() != w.numel() or e8m0_out.numel() != rows * (K // MX_BLOCK):
        raise ValueError("output sizes do not match w")
    _run("mx8_quantize", [w, q_out, e8m0_out], lib().mx8_quantize, w.data_ptr(), rows, K,
         q_out.data_ptr(), e8m0_out.data_ptr(), _stream(w, stream), stream=stream)
    return q_out, e8m0_out


def fp8q_sum_f32(parts: Sequence[torch.Tensor], out_dtype=torch.float32,
                 out: Optional[torch.Tensor] = None, stream=None):
    """Ordered fp32 sum of k arrays (the naive dequantize-then-reduce's second pass)."""
    k = len(parts)
    if k < 1 or k > MAX_PEERS:
        raise ValueError("need 1 .. %d parts" % MAX_PEERS)
    n = parts[0].numel()
    for i, p in enumerate(parts):
        _need(p, torch.float32, "parts[%d]" % i)
        if p.numel() != n:
            raise ValueError("part %d has the wrong size" % i)
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=parts[0].device)
    _need(out, out_dtype, "out")
    if out.numel() != n:
        raise ValueError("out must hold n values")
    _run("fp8q_sum_f32", [*parts, out], lib().fp8q_sum_f32, _ptrs(parts), k, n, out.data_ptr(),
         _out_code(out_dtype), _stream(parts[0], stream), stream=stream)
    return out


def fp8q_dequant_reduce_requantize(qs: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
                                   fmt_in: int = E4M3, fmt_out: Optional[int] = None,
                                   q_out: Optional[torch.Tensor] = None,
                                   scales_out: Optional[torch.Tensor] = None, stream=None):
    """Fused reduce of k peers, then block-128 requantize of the fp32 sums."""
    if fmt_out is None:
        fmt_out = fmt_in
    k = len(qs)
    if k < 1 or k != len(scales) or k > MAX_PEERS:
        raise ValueError("need 1 .. %d code tensors and as many scale tensors" % MAX_PEERS)
    n = qs[0].numel()
    for i, (q, s) in enumerate(zip(qs, scales)):
        _need(q, torch.uint8, "qs[%d]" % i)
        _need(s, torch.float32, "scales[%d]" % i)
        if q.numel() != n or s.numel() < num_scales(n):
            raise ValueError("peer %d has the wrong size" % i)
    if q_out is None:
        q_out = torch.empty(n, dtype=torch.uint8, device=qs[0].device)
    if scales_out is None:
        scales_out = torch.empty(num_scales(n), dtype=torch.float32, device=qs[0].device)
    _need(q_out, torch.uint8, "q_out")
    _need(scales_out, torch.float32, "scales_out")
    if q_out.numel() != n or scales_out.numel() != num_scales(n):
        raise ValueError("q_out must hold n codes and scales_out ceil(n/128) scales")
    _run("fp8q_dequant_reduce_requantize", [*qs, *scales, q_out, scales_out],
         lib().fp8q_dequant_reduce_requantize, _ptrs(qs), _ptrs(scales), k, n, _fmt(fmt_in),
         _fmt(fmt_out), q_out.data_ptr(), scales_out.data_ptr(), _stream(qs[0], stream), stream=stream)
    return q_out, scales_out


def mx8_dequant_reduce(qs: Sequence[torch.Tensor], e8m0s: Sequence[torch.Tensor],
                       out_dtype=torch.float32, out: Optional[torch.Tensor] = None, stream=None):
    """Sum over k MXFP8 shards of dec_e4m3(q) * 2^(code - 127), in peer order."""
    k = len(qs)
    if k < 1 or k != len(e8m0s) or k > MAX_PEERS:
        raise ValueError("need 1 .. %d code tensors and as many E8M0 tensors" % MAX_PEERS)
    shape = qs[0].shape
    if len(shape) < 1 or shape[-1] % MX_BLOCK:
        raise ValueError("codes must be [..., K] with K a multiple of 32")
    K = shape[-1]
    rows = qs[0].numel() // K if K else 0
    for i, (q, e) in enumerate(zip(qs, e8m0s)):
        _need(q, torch.uint8, "qs[%d]" % i)
        _need(e, torch.uint8, "e8m0s[%d]" % i)
        if q.shape != shape or e.numel() != rows * (K // MX_BLOCK):
            raise ValueError("peer %d has the wrong size" % i)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=qs[0].device)
    _need(out, out_dtype, "out")
    if out.numel() != qs[0].numel():
        raise ValueError("out must hold rows * K values")
    _run("mx8_dequant_reduce", [*qs, *e8m0s, out], lib().mx8_dequant_reduce, _ptrs(qs),
         _ptrs(e8m0s), k, rows, K, out.data_ptr(), _out_code(out_dtype), _stream(qs[0], stream), stream=stream)
    return out


def mx8_dequantize(q: torch.Tensor, e8m0: torch.Tensor, out_dtype=torch.float32,
                   out: Optional[torch.Tensor] = None, stream=None):
    """dec_e4m3(q) * 2^(code - 127) per 32-element block along K."""
    _need(q, torch.uint8, "q")
    _need(e8m0, torch.uint8, "e8m0")
    if q.dim() < 1 or q.shape[-1] % MX_BLOCK:
        raise ValueError("codes must be [..., K] with K a multiple of 32")
    K = q.shape[-1]
    rows = q.numel() // K if K else 0
    if e8m0.numel() != rows * (K // MX_BLOCK):
        raise ValueError("e8m0 must hold rows * K / 32 bytes")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _need(out, out_dtype, "out")
    if out.numel() != q.numel():
        raise ValueError("out must hold rows * K values")
    _run("mx8_dequantize", [q, e8m0, out], lib().mx8_dequantize, q.data_ptr(), e8m0.data_ptr(),
         rows, K, out.data_ptr(), _out_code(out_dtype), _stream(q, stream), stream=stream)
    return out


def fp8q_quantize_tensorwise(x: torch.Tensor, fmt: int = E4M3, q_out: Optional[torch.Tensor] = None,
                             scale_out: Optional[torch.Tensor] = None, stream=None):
    """One fp32 scale for the whole tensor -> (q uint8 [n], scale f32 [1])."""
    _need(x, torch.bfloat16, "x")
    n = x.numel()
    if q_out is None:
        q_out = torch.empty(n, dtype=torch.uint8, device=x.device)
    if scale_out is None:
        scale_out = torch.empty(1, dtype=torch.float32, device=x.device)
    _need(q_out, torch.uint8, "q_out")
    _need(scale_out, torch.float32, "scale_out")
    if q_out.numel() != n or scale_out.numel() != 1:
        raise ValueError("q_out must hold n codes and scale_out one scale")
    _run("fp8q_quantize_tensorwise", [x, q_out, scale_out], lib().fp8q_quantize_tensorwise,
         x.data_ptr(), n, _fmt(fmt), q_out.data_ptr(), scale_out.data_ptr(), _stream(x, stream), stream=stream)
    return q_out, scale_out
