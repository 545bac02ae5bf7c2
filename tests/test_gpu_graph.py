"""The codec's entry points allocate nothing and launch only kernels, so a
caller can capture them in a HIP graph (torch.cuda.CUDAGraph).  Replays must
equal the eager result every time, with eager work and synchronisations in
between (tensorwise quantize included: it reuses its scale slot as the amax
slot, which must be reset on every replay)."""
import pytest
import torch

import dequantize_reduce_transfer_amd as fq
from dequantize_reduce_transfer_amd import workloads
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    dev = require_gpu()
    n = 128 * 4000 + 77
    xs = [workloads.tiny_gradient(p, n=n, zero_block=None).to(dev) for p in range(4)]
    qs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(4)]
    ss = [torch.empty(fq.num_scales(n), dtype=torch.float32, device=dev) for _ in range(4)]
    y = torch.empty(n, dtype=torch.float32, device=dev)
    rq = torch.empty(n, dtype=torch.uint8, device=dev)
    rs = torch.empty(fq.num_scales(n), dtype=torch.float32, device=dev)
    tq = torch.empty(n, dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    w = workloads.kaiming_uniform((64, 512), seed=3).to(dev)
    mq = torch.empty((64, 512), dtype=torch.uint8, device=dev)
    me = torch.empty((64, 16), dtype=torch.uint8, device=dev)
    my = torch.empty((64, 512), dtype=torch.bfloat16, device=dev)

    def work():
        for p in range(4):
            fq.fp8q_quantize(xs[p], fq.E4M3, q_out=qs[p], scales_out=ss[p])
        fq.fp8q_dequant_reduce(qs, ss, fq.E4M3, out=y)
        fq.fp8q_dequant_reduce_requantize(qs, ss, fq.E4M3, fq.E5M2, q_out=rq, scales_out=rs)
        fq.fp8q_quantize_tensorwise(xs[1], fq.E5M2, q_out=tq, scale_out=ts)
        fq.mx8_quantize(w, q_out=mq, e8m0_out=me)
        fq.mx8_dequantize(mq, me, out_dtype=torch.bfloat16, out=my)

    outs = [y, rq, rs, tq, ts, mq, me, my] + qs + ss

    def snapshot():
        torch.cuda.synchronize()
        return [o.clone() for o in outs]

    work()
    eager = snapshot()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for r in range(4):
        for o in outs:                      # eager work between replays
            o.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for a, b in zip(got, eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "replay %d differs" % r
