"""The C-ABI library: it loads, exports every symbol include/fp8q.h declares,
and rejects every bad request on the host before any launch.

These tests never reach a kernel launch: each call fails validation first.
They are skipped when a GPU is visible, so that a validation bug could never
turn a host pointer into a launch there.
"""
import ctypes
import os
import re

import pytest
import torch

import dequantize_reduce_transfer_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

OK, ERR_NULL, ERR_ARG, ERR_ALIGN, ERR_OVERLAP, ERR_HIP = range(6)

no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="host-only validation tests; a GPU is visible")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^FP8Q_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert _declared() == sorted(fq.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fq.lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert fq.fp8q_abi_version() == 1
    text = open(HEADER).read()
    assert re.search(r"#define FP8Q_ABI_VERSION 1\b", text)
    for s in range(6):
        assert fq.fp8q_status_str(s).startswith("FP8Q_")
    assert "unknown" in fq.fp8q_status_str(99)


class Buf:
    """Host memory whose addresses stand in for device pointers; validation
    only compares addresses, it never dereferences them."""

    def __init__(self, nbytes, offset=0):
        self.raw = ctypes.create_string_buffer(nbytes + 64)
        base = ctypes.addressof(self.raw)
        self.addr = (base + 15) // 16 * 16 + offset


def P(x):
    return ctypes.c_void_p(x)


def PP(*addrs):
    return (ctypes.c_void_p * len(addrs))(*addrs)


@no_gpu
def test_quantize_validation():
    L = fq.lib()
    x, q, s = Buf(2 * 1000), Buf(1000), Buf(4 * 8)
    assert L.fp8q_quantize(P(x.addr), 1000, 2, P(q.addr), P(s.addr), None) == ERR_ARG
    assert L.fp8q_quantize(P(x.addr), 1000, -1, P(q.addr), P(s.addr), None) == ERR_ARG
    assert L.fp8q_quantize(None, 0, 0, None, None, None) == OK            # n == 0: no-op
    assert L.fp8q_quantize(P(x.addr), (1 << 40) + 1, 0, P(q.addr), P(s.addr), None) == ERR_ARG
    assert L.fp8q_quantize(None, 1000, 0, P(q.addr), P(s.addr), None) == ERR_NULL
    assert L.fp8q_quantize(P(x.addr), 1000, 0, None, P(s.addr), None) == ERR_NULL
    assert L.fp8q_quantize(P(x.addr), 1000, 0, P(q.addr), None, None) == ERR_NULL
    assert L.fp8q_quantize(P(x.addr + 2), 1000, 0, P(q.addr), P(s.addr), None) == ERR_ALIGN
    assert L.fp8q_quantize(P(x.addr), 1000, 0, P(q.addr + 8), P(s.addr), None) == ERR_ALIGN
    assert L.fp8q_quantize(P(x.addr), 1000, 0, P(q.addr), P(s.addr + 2), None) == ERR_ALIGN
    # q inside x, scales inside q, scales inside x
    assert L.fp8q_quantize(P(x.addr), 1000, 0, P(x.addr + 1008), P(s.addr), None) == ERR_OVERLAP
    assert L.fp8q_quantize(P(x.addr), 1000, 0, P(q.addr), P(q.addr + 996), None) == ERR_OVERLAP
    assert L.fp8q_quantize(P(x.addr), 1000, 0, P(q.addr), P(x.addr + 1996), None) == ERR_OVERLAP


@no_gpu
def test_dequantize_validation():
    L = fq.lib()
    q, s, y = Buf(1000), Buf(32), Buf(4 * 1000)
    assert L.fp8q_dequantize(P(q.addr), P(s.addr), 1000, 3, P(y.addr), 0, None) == ERR_ARG
    assert L.fp8q_dequantize(P(q.addr), P(s.addr), 1000, 0, P(y.addr), 2, None) == ERR_ARG
    assert L.fp8q_dequantize(None, None, 0, 0, None, 0, None) == OK
    assert L.fp8q_dequantize(None, P(s.addr), 1000, 0, P(y.addr), 0, None) == ERR_NULL
    assert L.fp8q_dequantize(P(q.addr), None, 1000, 0, P(y.addr), 0, None) == ERR_NULL
    assert L.fp8q_dequantize(P(q.addr), P(s.addr), 1000, 0, None, 0, None) == ERR_NULL
    assert L.fp8q_dequantize(P(q.addr + 4), P(s.addr), 1000, 0, P(y.addr), 0, None) == ERR_ALIGN
    assert L.fp8q_dequantize(P(q.addr), P(s.addr), 1000, 0, P(y.addr + 8), 1, None) == ERR_ALIGN
    assert L.fp8q_dequantize(P(q.addr), P(s.addr), 1000, 0, P(q.addr + 496), 1, None) == ERR_OVERLAP
    assert L.fp8q_dequantize(P(q.addr), P(y.addr + 3996), 1000, 0, P(y.addr), 0, None) == ERR_OVERLAP


@no_gpu
def test_dequant_reduce_validation():
    L = fq.lib()
    n = 4096
    qs = [Buf(n) for _ in range(17)]
    ss = [Buf(4 * 32) for _ in range(17)]
    y = Buf(4 * n)
    qa = PP(*[b.addr for b in qs])
    sa = PP(*[b.addr for b in ss])
    assert L.fp8q_dequant_reduce(qa, sa, 0, n, 0, P(y.addr), 0, None) == ERR_ARG
    assert L.fp8q_dequant_reduce(qa, sa, 17, n, 0, P(y.addr), 0, None) == ERR_ARG
    assert L.fp8q_dequant_reduce(qa, sa, 4, n, 5, P(y.addr), 0, None) == ERR_ARG
    assert L.fp8q_dequant_reduce(qa, sa, 4, n, 0, P(y.addr), 7, None) == ERR_ARG
    assert L.fp8q_dequant_reduce(None, None, 4, 0, 0, None, 0, None) == OK
    assert L.fp8q_dequant_reduce(None, sa, 4, n, 0, P(y.addr), 0, None) == ERR_NULL
    assert L.fp8q_dequant_reduce(qa, sa, 4, n, 0, None, 0, None) == ERR_NULL
    qa_null = PP(qs[0].addr, qs[1].addr, 0, qs[3].addr)
    assert L.fp8q_dequant_reduce(qa_null, sa, 4, n, 0, P(y.addr), 0, None) == ERR_NULL
    qa_mis = PP(qs[0].addr, qs[1].addr + 1, qs[2].addr, qs[3].addr)
    assert L.fp8q_dequant_reduce(qa_mis, sa, 4, n, 0, P(y.addr), 0, None) == ERR_ALIGN
    sa_mis = PP(ss[0].addr, ss[1].addr, ss[2].addr + 2, ss[3].addr)
    assert L.fp8q_dequant_reduce(qa, sa_mis, 4, n, 0, P(y.addr), 0, None) == ERR_ALIGN
    # output overlapping peer 3's codes, then peer 2's scales
    qa_ov = PP(qs[0].addr, qs[1].addr, qs[2].addr, y.addr + 4 * n - 16)
    assert L.fp8q_dequant_reduce(qa_ov, sa, 4, n, 0, P(y.addr), 0, None) == ERR_OVERLAP
    sa_ov = PP(ss[0].addr, ss[1].addr, y.addr, ss[3].addr)
    assert L.fp8q_dequant_reduce(qa, sa_ov, 4, n, 0, P(y.addr), 0, None) == ERR_OVERLAP
    # peers may share inputs (read-only); only outputs must be disjoint --
    # checked through the bf16 output size: a bf16 output of n values ends
    # at 2n bytes, so codes placed right after it do not overlap
    qa_after = PP(y.addr + 2 * n, qs[1].addr, qs[2].addr, qs[3].addr)
    assert L.fp8q_dequant_reduce(qa_after, sa, 4, n, 0, P(y.addr), 0, None) == ERR_OVERLAP
    qa_after_bad_k = PP(y.addr + 2 * n, qs[1].addr)
    assert L.fp8q_dequant_reduce(qa_after_bad_k, sa, 0, n, 0, P(y.addr), 1, None) == ERR_ARG


@no_gpu
def test_mx8_validation():
    L = fq.lib()
    rows, K = 64, 256
    w, q, e = Buf(2 * rows * K), Buf(rows * K), Buf(rows * K // 32)
    assert L.mx8_quantize(P(w.addr), rows, 48, P(q.addr), P(e.addr), None) == ERR_ARG
    assert L.mx8_quantize(P(w.addr), rows, 33, P(q.addr), P(e.addr), None) == ERR_ARG
    assert L.mx8_quantize(None, 0, K, None, None, None) == OK
    assert L.mx8_quantize(None, rows, 0, None, None, None) == OK
    assert L.mx8_quantize(P(w.addr), 1 << 40, 64, P(q.addr), P(e.addr), None) == ERR_ARG
    assert L.mx8_quantize(None, rows, K, P(q.addr), P(e.addr), None) == ERR_NULL
    assert L.mx8_quantize(P(w.addr), rows, K, P(q.addr), None, None) == ERR_NULL
    assert L.mx8_quantize(P(w.addr + 8), rows, K, P(q.addr), P(e.addr), None) == ERR_ALIGN
    assert L.mx8_quantize(P(w.addr), rows, K, P(q.addr + 4), P(e.addr), None) == ERR_ALIGN
    assert L.mx8_quantize(P(w.addr), rows, K, P(w.addr + 2 * rows * K - 16), P(e.addr), None) == ERR_OVERLAP
    assert L.mx8_quantize(P(w.addr), rows, K, P(q.addr), P(q.addr + 100), None) == ERR_OVERLAP


@no_gpu
def test_sum_validation():
    L = fq.lib()
    n = 1000
    parts = [Buf(4 * n) for _ in range(3)]
    y = Buf(4 * n)
    pa = PP(*[b.addr for b in parts])
    assert L.fp8q_sum_f32(pa, 0, n, P(y.addr), 0, None) == ERR_ARG
    assert L.fp8q_sum_f32(pa, 3, n, P(y.addr), 2, None) == ERR_ARG
    assert L.fp8q_sum_f32(None, 3, 0, None, 0, None) == OK
    assert L.fp8q_sum_f32(pa, 3, n, None, 0, None) == ERR_NULL
    assert L.fp8q_sum_f32(pa, 3, n, P(y.addr + 4), 0, None) == ERR_ALIGN
    pa_ov = PP(parts[0].addr, y.addr + 16, parts[2].addr)
    assert L.fp8q_sum_f32(pa_ov, 3, n, P(y.addr), 0, None) == ERR_OVERLAP


def test_binding_rejects_cpu_tensors_before_the_library():
    x = torch.zeros(256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fq.fp8q_quantize(x)
    with pytest.raises(TypeError):
        fq.fp8q_quantize(torch.zeros(256, dtype=torch.float32))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(fq, "_lib", None)
    monkeypatch.setattr(fq, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fq.lib()


@no_gpu
def test_requantize_validation():
    L = fq.lib()
    n = 4096
    qs = [Buf(n) for _ in range(4)]
    ss = [Buf(4 * 32) for _ in range(4)]
    qo, so = Buf(n), Buf(4 * 32)
    qa = PP(*[b.addr for b in qs])
    sa = PP(*[b.addr for b in ss])
    f = L.fp8q_dequant_reduce_requantize
    assert f(qa, sa, 4, n, 0, 2, P(qo.addr), P(so.addr), None) == ERR_ARG
    assert f(qa, sa, 0, n, 0, 0, P(qo.addr), P(so.addr), None) == ERR_ARG
    assert f(qa, sa, 17, n, 0, 0, P(qo.addr), P(so.addr), None) == ERR_ARG
    assert f(None, None, 4, 0, 0, 1, None, None, None) == OK
    assert f(qa, sa, 4, n, 0, 1, None, P(so.addr), None) == ERR_NULL
    assert f(qa, sa, 4, n, 0, 1, P(qo.addr), None, None) == ERR_NULL
    assert f(qa, sa, 4, n, 0, 1, P(qo.addr + 4), P(so.addr), None) == ERR_ALIGN
    assert f(qa, sa, 4, n, 0, 1, P(qo.addr), P(so.addr + 1), None) == ERR_ALIGN
    assert f(qa, sa, 4, n, 0, 1, P(qo.addr), P(qo.addr + n - 16), None) == ERR_OVERLAP
    # in-place over a peer's codes or scales is rejected
    assert f(qa, sa, 4, n, 0, 1, P(qs[2].addr), P(so.addr), None) == ERR_OVERLAP
    assert f(qa, sa, 4, n, 0, 1, P(qo.addr), P(ss[3].addr), None) == ERR_OVERLAP


@no_gpu
def test_mx8_receiver_validation():
    L = fq.lib()
    rows, K = 16, 256
    n = rows * K
    q, e, y = Buf(n), Buf(n // 32), Buf(4 * n)
    assert L.mx8_dequantize(P(q.addr), P(e.addr), rows, 48, P(y.addr), 0, None) == ERR_ARG
    assert L.mx8_dequantize(P(q.addr), P(e.addr), rows, K, P(y.addr), 3, None) == ERR_ARG
    assert L.mx8_dequantize(None, None, 0, K, None, 0, None) == OK
    assert L.mx8_dequantize(None, P(e.addr), rows, K, P(y.addr), 0, None) == ERR_NULL
    assert L.mx8_dequantize(P(q.addr), None, rows, K, P(y.addr), 0, None) == ERR_NULL
    assert L.mx8_dequantize(P(q.addr), P(e.addr), rows, K, None, 0, None) == ERR_NULL
    assert L.mx8_dequantize(P(q.addr + 8), P(e.addr), rows, K, P(y.addr), 0, None) == ERR_ALIGN
    assert L.mx8_dequantize(P(q.addr), P(e.addr + 3), rows, K, P(y.addr + 4), 0, None) == ERR_ALIGN
    assert L.mx8_dequantize(P(q.addr), P(y.addr + 4 * n - 8), rows, K, P(y.addr), 0, None) == ERR_OVERLAP
    qa = PP(q.addr, q.addr)
    ea = PP(e.addr, e.addr + 1)       # E8M0 arrays need no alignment
    assert L.mx8_dequant_reduce(qa, ea, 0, rows, K, P(y.addr), 0, None) == ERR_ARG
    assert L.mx8_dequant_reduce(qa, ea, 17, rows, K, P(y.addr), 0, None) == ERR_ARG
    assert L.mx8_dequant_reduce(qa, PP(e.addr, 0), 2, rows, K, P(y.addr), 0, None) == ERR_NULL
    assert L.mx8_dequant_reduce(PP(q.addr, y.addr), ea, 2, rows, K, P(y.addr), 1, None) == ERR_OVERLAP


@no_gpu
def test_tensorwise_validation():
    L = fq.lib()
    n = 1000
    x, q, s = Buf(2 * n), Buf(n), Buf(16)
    f = L.fp8q_quantize_tensorwise
    assert f(P(x.addr), n, 9, P(q.addr), P(s.addr), None) == ERR_ARG
    assert f(None, 0, 0, None, None, None) == OK
    assert f(P(x.addr), (1 << 40) + 1, 0, P(q.addr), P(s.addr), None) == ERR_ARG
    assert f(P(x.addr), n, 0, P(q.addr), None, None) == ERR_NULL
    assert f(P(x.addr + 2), n, 0, P(q.addr), P(s.addr), None) == ERR_ALIGN
    assert f(P(x.addr), n, 0, P(q.addr), P(s.addr + 2), None) == ERR_ALIGN
    assert f(P(x.addr), n, 0, P(q.addr), P(x.addr + 1000), None) == ERR_OVERLAP
    assert f(P(x.addr), n, 0, P(q.addr), P(q.addr + 996), None) == ERR_OVERLAP


# ---------------------------------------------------------------------------
# Accepted calls.  The host-check build of the library (csrc/api.hip compiled
# host-only, with tests/native/abi_stub_launchers.cpp in place of the
# kernels) records each launch instead of enqueueing it, so a valid call can
# run on a machine without a GPU: it must reach its launcher exactly once,
# with the caller's n and k, and every rejected call above must reach none.
# tests/test_abi_sanitized.py runs this whole file against that build under
# AddressSanitizer and UndefinedBehaviorSanitizer.

def _stub():
    L = fq.lib()
    if not hasattr(L, "fp8q_stub_calls"):
        pytest.skip("needs the host-check build of the library (FP8Q_LIB)")
    L.fp8q_stub_calls.restype = ctypes.c_long
    L.fp8q_stub_last.restype = ctypes.c_char_p
    L.fp8q_stub_last_n.restype = ctypes.c_ulonglong
    L.fp8q_stub_last_k.restype = ctypes.c_int
    return L


def _expect_launch(L, status, name, n, k=1):
    before = L.fp8q_stub_calls()
    assert status() == OK
    assert L.fp8q_stub_calls() == before + 1
    assert L.fp8q_stub_last().decode() == name
    assert L.fp8q_stub_last_n() == n and L.fp8q_stub_last_k() == k


def _expect_no_launch(L, status, want):
    before = L.fp8q_stub_calls()
    assert status() == want
    assert L.fp8q_stub_calls() == before


def test_accepted_calls_reach_their_launcher_once():
    L = _stub()
    n = 1000
    x, q, s = Buf(2 * n), Buf(n), Buf(4 * 8)
    _expect_launch(L, lambda: L.fp8q_quantize(P(x.addr), n, 1, P(q.addr), P(s.addr), None),
                   "quantize", n)
    _expect_launch(L, lambda: L.fp8q_quantize_tensorwise(P(x.addr), n, 0, P(q.addr), P(s.addr),
                                                         None), "quantize_tensorwise", n)
    y = Buf(4 * n)
    _expect_launch(L, lambda: L.fp8q_dequantize(P(q.addr), P(s.addr), n, 0, P(y.addr), 1, None),
                   "dequantize", n)
    for k in (1, 2, 16):
        qs = [Buf(n) for _ in range(k)]
        ss = [Buf(4 * 8) for _ in range(k)]
        qa, sa = PP(*[b.addr for b in qs]), PP(*[b.addr for b in ss])
        _expect_launch(L, lambda: L.fp8q_dequant_reduce(qa, sa, k, n, 1, P(y.addr), 0, None),
                       "dequantize" if k == 1 else "dequant_reduce", n, k)
        qo, so = Buf(n), Buf(4 * 8)
        _expect_launch(L, lambda: L.fp8q_dequant_reduce_requantize(
            qa, sa, k, n, 0, 1, P(qo.addr), P(so.addr), None), "reduce_requantize", n, k)
        parts = [Buf(4 * n) for _ in range(k)]
        pa = PP(*[b.addr for b in parts])
        _expect_launch(L, lambda: L.fp8q_sum_f32(pa, k, n, P(y.addr), 1, None), "sum_f32", n, k)
    rows, K = 7, 96
    w, qm, e = Buf(2 * rows * K), Buf(rows * K), Buf(rows * K // 32)
    _expect_launch(L, lambda: L.mx8_quantize(P(w.addr), rows, K, P(qm.addr), P(e.addr + 1), None),
                   "mx8_quantize", rows * K)
    ym = Buf(4 * rows * K)
    _expect_launch(L, lambda: L.mx8_dequantize(P(qm.addr), P(e.addr + 3), rows, K, P(ym.addr), 0,
                                               None), "mx8_dequantize", rows * K)
    qa, ea = PP(qm.addr, qm.addr), PP(e.addr, e.addr + 1)
    _expect_launch(L, lambda: L.mx8_dequant_reduce(qa, ea, 2, rows, K, P(ym.addr), 1, None),
                   "mx8_dequant_reduce", rows * K, 2)


def test_rejected_and_empty_calls_reach_no_launcher():
    L = _stub()
    n = 1000
    x, q, s, y = Buf(2 * n), Buf(n), Buf(4 * 8), Buf(4 * n)
    _expect_no_launch(L, lambda: L.fp8q_quantize(None, 0, 0, None, None, None), OK)
    _expect_no_launch(L, lambda: L.fp8q_quantize(P(x.addr), n, 0, P(x.addr + 16), P(s.addr), None),
                      ERR_OVERLAP)
    _expect_no_launch(L, lambda: L.fp8q_quantize(P(x.addr + 2), n, 0, P(q.addr), P(s.addr), None),
                      ERR_ALIGN)
    _expect_no_launch(L, lambda: L.fp8q_dequantize(P(q.addr), P(s.addr), n, 0, None, 0, None),
                      ERR_NULL)
    qa, sa = PP(q.addr, q.addr), PP(s.addr, s.addr)
    _expect_no_launch(L, lambda: L.fp8q_dequant_reduce(qa, sa, 2, n, 0, P(y.addr), 9, None),
                      ERR_ARG)
    _expect_no_launch(L, lambda: L.fp8q_dequant_reduce_requantize(
        qa, sa, 2, n, 0, 0, P(q.addr), P(s.addr), None), ERR_OVERLAP)
    _expect_no_launch(L, lambda: L.mx8_quantize(P(x.addr), 10, 48, P(q.addr), P(s.addr), None),
                      ERR_ARG)
    _expect_no_launch(L, lambda: L.mx8_dequant_reduce(qa, sa, 17, 10, 64, P(y.addr), 0, None),
                      ERR_ARG)
    _expect_no_launch(L, lambda: L.fp8q_sum_f32(PP(y.addr), 1, n, P(y.addr), 0, None), ERR_OVERLAP)
