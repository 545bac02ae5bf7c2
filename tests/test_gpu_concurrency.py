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
