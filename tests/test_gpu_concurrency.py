"""The library keeps no state between calls: several host threads, each on
its own HIP stream, run quantize -> reduce -> requantize -> MXFP8 chains at
the same time and every result matches the same chain run alone."""
import threading

import pytest
import torch

import dequantize_reduce_transfer_amd as fq
from dequantize_reduce_transfer_amd import workloads
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def _chain(x, w, k):
    q, s = fq.fp8q_quantize(x, fq.E4M3)
    n = x.numel() // k // 128 * 128
    qs = [q[p * n:(p + 1) * n] for p in range(k)]
    ss = [s[p * n // 128:(p + 1) * n // 128] for p in range(k)]
    y = fq.fp8q_dequant_reduce(qs, ss, fq.E4M3, out_dtype=torch.bfloat16)
    rq, rs = fq.fp8q_dequant_reduce_requantize(qs, ss, fq.E4M3, fq.E5M2)
    wq, we = fq.mx8_quantize(w)
    return [q, s, y, rq, rs, wq, we]


def test_threads_on_separate_streams_match_serial():
    dev = require_gpu()
    jobs = []
    for j in range(4):
        x = workloads.segmented_gradient((1 << 22) + 128 * j, seed=40 + j, device=dev,
                                         segment=1 << 20)
        w = workloads.kaiming_uniform((256, 1024), seed=50 + j, device=dev)
        jobs.append((x, w, 2 + 2 * j))
    want = [_chain(*a) for a in jobs]
    torch.cuda.synchronize()

    got = [None] * len(jobs)
    errors = []

    def worker(i):
        try:
            st = torch.cuda.Stream(device=dev)
            st.wait_stream(torch.cuda.default_stream(dev))
            with torch.cuda.stream(st):
                for _ in range(10):
                    res = _chain(*jobs[i])
                st.synchronize()
            got[i] = res
        except Exception as e:          # surfaced below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(len(jobs)):
        for a, b in zip(got[i], want[i]):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), i


def _chain_on(x, w, k, st):
    """_chain with every call given the stream explicitly (no stream context)."""
    q, s = fq.fp8q_quantize(x, fq.E4M3, stream=st)
    n = x.numel() // k // 128 * 128
    qs = [q[p * n:(p + 1) * n] for p in range(k)]
    ss = [s[p * n // 128:(p + 1) * n // 128] for p in range(k)]
    y = fq.fp8q_dequant_reduce(qs, ss, fq.E4M3, out_dtype=torch.bfloat16, stream=st)
    rq, rs = fq.fp8q_dequant_reduce_requantize(qs, ss, fq.E4M3, fq.E5M2, stream=st)
    wq, we = fq.mx8_quantize(w, stream=st)
    return [q, s, y, rq, rs, wq, we]


def test_explicit_stream_argument_matches_current_stream():
    """Outputs the binding allocates for a call on a caller-named stream stay
    that call's while the stream runs, even as the current stream allocates
    and frees memory meanwhile; the results equal the same chain run on the
    current stream."""
    dev = require_gpu()
    x = workloads.segmented_gradient((1 << 22) + 128, seed=60, device=dev, segment=1 << 20)
    w = workloads.kaiming_uniform((256, 1024), seed=61, device=dev)
    want = _chain(x, w, 4)
    want_dq = fq.fp8q_dequantize(want[0], want[1], fq.E4M3)
    want_mx = fq.mx8_dequantize(want[5], want[6], out_dtype=torch.bfloat16)
    want_tw = fq.fp8q_quantize_tensorwise(x, fq.E5M2)
    torch.cuda.synchronize()

    st = torch.cuda.Stream(device=dev)
    st.wait_stream(torch.cuda.current_stream(dev))
    got = _chain_on(x, w, 4, st)
    got_dq = fq.fp8q_dequantize(got[0], got[1], fq.E4M3, stream=st)
    got_mx = fq.mx8_dequantize(got[5], got[6], out_dtype=torch.bfloat16, stream=st)
    got_tw = fq.fp8q_quantize_tensorwise(x, fq.E5M2, stream=st)
    for _ in range(8):                  # allocator churn on the current stream
        junk = torch.full((1 << 22,), 7, dtype=torch.uint8, device=dev)
        del junk
    st.synchronize()
    torch.cuda.synchronize()
    pairs = list(zip(got, want)) + [(got_dq, want_dq), (got_mx, want_mx)]
    pairs += list(zip(got_tw, want_tw))
    for i, (a, b) in enumerate(pairs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), i


def test_released_outputs_are_not_reused_while_the_named_stream_runs():
    """Codes and scales the binding allocates for a call on a named stream
    are released by the caller while a later call queued on that stream has
    yet to read them; memory of the same size allocated and overwritten on
    the current stream meanwhile must not be theirs.  A few milliseconds of
    work on the named stream sit between the call that writes them and the
    call that reads them, so the current stream's writes land in between."""
    dev = require_gpu()
    n = (1 << 22) + 128 * 3
    x = workloads.segmented_gradient(n, seed=70, device=dev, segment=1 << 20)
    busy = workloads.sweep_payload(1 << 28, seed=71, device=dev)          # 2^27 bf16
    q0, s0 = fq.fp8q_quantize(x, fq.E4M3)
    want = fq.fp8q_dequantize(q0, s0, fq.E4M3)
    torch.cuda.synchronize()

    st = torch.cuda.Stream(device=dev)
    st.wait_stream(torch.cuda.current_stream(dev))
    bq = torch.empty(busy.numel(), dtype=torch.uint8, device=dev)
    bs = torch.empty(fq.num_scales(busy.numel()), dtype=torch.float32, device=dev)
    q, s = fq.fp8q_quantize(x, fq.E4M3, stream=st)
    for _ in range(40):                 # a few ms of work on st between the two calls
        fq.fp8q_quantize(busy, fq.E4M3, q_out=bq, scales_out=bs, stream=st)
    got = fq.fp8q_dequantize(q, s, fq.E4M3, stream=st)
    del q, s                            # released before st has read them
    junk_q = torch.full((n,), 0x7E, dtype=torch.uint8, device=dev)
    junk_s = torch.full((fq.num_scales(n),), 1.0e30, dtype=torch.float32, device=dev)
    st.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    del junk_q, junk_s, bq, bs, busy
