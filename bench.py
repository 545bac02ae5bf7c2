"""Benchmark of the FP8 wire codec's hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step is one pass of the whole hot path over the workload, all inputs
already resident in HBM:
  1. block-128 e4m3 quantize of the Pi0.5-scale bf16 gradient
     (3.5e9 elements, ~7 GB; 27,343,750 fp32 scales);
  2. fused dequant-reduce of 8 peer shards of 437,500,000 elements into fp32;
     the shards are 8 block-aligned slices (stride 437,499,904 elements) of
     step 1's codes and scales, so every shard is real quantized gradient
     and every dispatch of a timed kernel has the same size;
  3. MXFP8 quantize of one Qwen3-30B-A3B-shaped MoE layer (128 experts:
     gate and up [768, 2048], down [2048, 768]; three launches).
`value` is the step's bf16-equivalent bytes (2 B per quantized element, 2 B
per element of every reduced peer) divided by the step time.

Per-launch kernel times come from HIP events recorded on the stream the
kernels run on (torch's current stream); the roofline figure uses the
dominant kernel (the 7 GB quantize) with its algorithmic HBM bytes
(2 + 1 + 4/128 B per element).  Side figures (not in the step): the
dequantize alone, and the naive dequantize-then-sum path that the fused
kernel replaces.  The CPU baseline times the oracle (plain C, run on
independent block-aligned pieces from a pool of host threads, and again on
one thread) on a bounded sample of the same workload.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quantize & dequant-reduce GB/s (bf16-equiv) and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
QUANT_BYTES_PER_ELEM = 2 + 1 + 4 / 128
MX_BYTES_PER_ELEM = 2 + 1 + 1 / 32
PROFILE_DIR = os.path.join(ROOT, "profiles")
QUANT_KERNEL_SRCS = [os.path.join(ROOT, "dequantize_reduce_transfer_amd", "csrc", f)
                     for f in ("quantize.hip", "fp8q_device.h", "launch.h")]


_T0 = time.perf_counter()


def log(msg):
    sys.stderr.write("[bench %6.1fs] %s\n" % (time.perf_counter() - _T0, msg))
    sys.stderr.flush()


def reduce_bytes_per_elem(k, out_bytes):
    return k * (1 + 4 / 128) + out_bytes


def source_digest(paths):
    """SHA-256 of the kernel's sources with comments and whitespace removed,
    so that only a change to the code itself invalidates measured counters."""
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def read_traffic(kernel_srcs):
    """HBM traffic per dispatch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, "quantize_pi05_e4m3_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                vals[parts[0]] = parts[1]
    if vals.get("source_sha256") != source_digest(kernel_srcs):
        return None
    try:
        return float(vals["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events around each launch on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def mean_ms(self, name):
        ev = self.pairs.get(name, [])
        return sum(a.elapsed_time(b) for a, b in ev) / max(1, len(ev))

    def spread_us(self, name):
        """Median and minimum launch time in microseconds."""
        v = sorted(a.elapsed_time(b) for a, b in self.pairs.get(name, []))
        if not v:
            return {}
        return {"us_median": round(v[len(v) // 2] * 1e3, 2), "us_min": round(v[0] * 1e3, 2)}

    def reset(self):
        self.pairs = {}


def _cpu_sample(x, peers, moe, frac):
    """Host copies of the first `frac` of every input of the step."""
    from dequantize_reduce_transfer_amd import workloads

    n_q = int(x.numel() * frac) // 128 * 128
    n_r = int(peers[0][0].numel() * frac) // 128 * 128
    e_mx = max(1, int(moe["gate"].shape[0] * frac))
    return {
        "x": workloads.bits(x[:n_q]),
        "qs": [q[:n_r].cpu().numpy() for q, _ in peers],
        "ss": [s[: n_r // 128].cpu().numpy() for _, s in peers],
        "ws": {k: workloads.bits(v[:e_mx]).reshape((-1, v.shape[-1])) for k, v in moe.items()},
        "n_q": n_q, "n_r": n_r, "e_mx": e_mx,
    }


def _piece(total, parts, multiple):
    """Piece length: total / parts rounded up to a multiple, at least one multiple."""
    per = -(-total // parts)
    return max(multiple, -(-per // multiple) * multiple)


def _cpu_pieces(smp, fmt, threads):
    """The sample's oracle calls, cut at block boundaries into about
    4 * `threads` independent pieces (one piece each when threads == 1).
    Each job is (what, call): `what` names the output the call's result
    belongs to, so the pieces can be put back together in order."""
    import oracle

    parts = 1 if threads == 1 else 4 * threads
    jobs = []
    xq = smp["x"]
    step = _piece(xq.size, parts, 128)
    for a in range(0, xq.size, step):
        jobs.append(("quantize", lambda a=a, m=step: oracle.quantize(xq[a:a + m], fmt)))
    n_r = smp["n_r"]
    step = _piece(n_r, parts, 128)
    for a in range(0, n_r, step):
        jobs.append(("dequant_reduce", lambda a=a, m=step: oracle.dequant_reduce(
            [q[a:a + m] for q in smp["qs"]], [s[a // 128:(a + m) // 128] for s in smp["ss"]], fmt)))
    for name, w in smp["ws"].items():
        rows = w.shape[0]
        step = _piece(rows, parts, 1)
        for a in range(0, rows, step):
            jobs.append(("mx8_" + name, lambda w=w, a=a, m=step: oracle.mx8_quantize(w[a:a + m])))
    return jobs


def cpu_baseline(smp, fmt, threads, runs=1):
    """The oracle, as it stands, on the sample; with threads > 1 the same
    calls run on independent block-aligned pieces from a thread pool (the
    oracle's C calls release the GIL), as an OpenMP loop over blocks would.
    The time is the median of `runs` runs.  Returns the record and the
    oracle's outputs of the first run, in order, keyed by output."""
    from concurrent.futures import ThreadPoolExecutor

    jobs = _cpu_pieces(smp, fmt, threads)
    times = []
    outputs = None
    for r in range(runs):
        t0 = time.perf_counter()
        if threads == 1:
            res = [j() for _, j in jobs]
        else:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                res = [f.result() for f in [ex.submit(j) for _, j in jobs]]
        times.append(time.perf_counter() - t0)
        if r == 0:
            outputs = {}
            for (what, _), o in zip(jobs, res):
                outputs.setdefault(what, []).append(o)
        del res
    dt = sorted(times)[len(times) // 2]
    k = len(smp["qs"])
    bf16_bytes = (2 * smp["n_q"] + 2 * k * smp["n_r"]
                  + sum(2 * w.size for w in smp["ws"].values()))
    rec = {
        "value": round(bf16_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("first %.4g of each input: quantize %d elements, dequant-reduce k=%d x %d "
                   "elements, mx8 %d experts of each of 3 tensors; %.2f s wall on %d host "
                   "thread%s, median of %d run%s" % (
                       smp["frac"], smp["n_q"], k, smp["n_r"], smp["e_mx"], dt, threads,
                       "" if threads == 1 else "s, block-aligned pieces", runs,
                       "" if runs == 1 else "s")),
    }
    return rec, outputs


# A one-GPU MI355X host here gives its GPU a share of 16 CPUs (worker pools
# are sized to that share, whatever the machine's own count is), so the
# oracle's thread pool is capped there; the record states the machine's
# count, the process's CPU set and the model next to the threads used.
HOST_THREAD_CAP = 16


def host_cpus():
    """The host's CPU count, the process's CPU set and the CPU model."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model}


def host_threads():
    """Host threads for the CPU baseline: the process's CPU set, at most
    HOST_THREAD_CAP (the host's CPU share for one GPU)."""
    return max(1, min(HOST_THREAD_CAP, host_cpus()["affinity_cpus"]))


def _sample_idx(nunits, count, seed, always=()):
    """Sampled unit indices: the first and last 64, `count` random ones and
    `always`."""
    import numpy as np

    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(min(64, nunits)), np.arange(max(0, nunits - 64), nunits),
                          rng.integers(0, nunits, count), np.asarray(always, dtype=np.int64)])
    return np.unique(idx[(idx >= 0) & (idx < nunits)])


def _host(torch, t):
    import numpy as np

    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def step_parity(torch, fmt, smp, outputs, x, q, s, qs, ss, y, moe, mx_out):
    """The step's own GPU outputs against the oracle.

    1. Every output the CPU baseline's sample covers (the first part of the
       quantized gradient, of the reduce's output, and of each MoE tensor),
       against the oracle outputs the baseline's first run produced.
    2. Sampled units across the whole of each output: 8192 random 128-blocks
       of the quantized gradient (plus the first and last 64 and the blocks
       that straddle its 25M-element segments), 16384 reduced elements (plus
       the last 300, the shard's 96-element last block among them) and 512
       rows of each MoE tensor.  Each sampled unit depends only on its own
       inputs, so the oracle runs on just those.
    Returns a summary; raises AssertionError on the first mismatch."""
    import numpy as np

    import oracle
    from dequantize_reduce_transfer_amd import workloads

    def same(got, want, what):
        got = np.ascontiguousarray(got).ravel()
        want = np.ascontiguousarray(want).ravel()
        if got.shape != want.shape or not np.array_equal(got, want):
            bad = np.nonzero(got != want)[0] if got.shape == want.shape else [-1]
            raise AssertionError("%s: %d mismatches vs the oracle (first at %s)"
                                 % (what, len(bad), list(bad[:3])))

    def f32(a):
        return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)

    n_q, n_r = smp["n_q"], smp["n_r"]
    q_o = np.concatenate([o[0] for o in outputs["quantize"]])
    s_o = np.concatenate([o[1] for o in outputs["quantize"]])
    same(_host(torch, q[:n_q]), q_o, "quantize codes (sample)")
    same(f32(_host(torch, s[:n_q // 128])), f32(s_o), "quantize scales (sample)")
    same(f32(_host(torch, y[:n_r])), f32(np.concatenate(outputs["dequant_reduce"])),
         "dequant-reduce fp32 (sample)")
    mx_rows = 0
    for name in moe:
        q_m = np.concatenate([o[0] for o in outputs["mx8_" + name]])
        e_m = np.concatenate([o[1] for o in outputs["mx8_" + name]])
        rows, K = q_m.shape
        same(_host(torch, mx_out[name][0].view(-1, K)[:rows]), q_m, "mx8 %s codes (sample)" % name)
        same(_host(torch, mx_out[name][1][:rows]), e_m, "mx8 %s e8m0 (sample)" % name)
        mx_rows += rows
    covered = {"quantize_elements": int(n_q), "reduce_elements": int(n_r), "mx8_rows": mx_rows}

    dev = q.device
    nb = x.numel() // 128
    seg = workloads.PI05_SEGMENT
    edges = [(j * seg) // 128 for j in range(1, x.numel() // seg)]
    idx = _sample_idx(nb, 8192, seed=1, always=edges)
    it = torch.from_numpy(idx).to(dev)
    qb, sb = oracle.quantize(_host(torch, x[:nb * 128].view(-1, 128)[it]).ravel(), fmt)
    same(_host(torch, q[:nb * 128].view(-1, 128)[it]), qb, "quantize codes (sampled blocks)")
    same(f32(_host(torch, s[it])), f32(sb), "quantize scales (sampled blocks)")

    n = y.numel()
    eidx = _sample_idx(n, 16384, seed=2, always=np.arange(n - 300, n))
    et = torch.from_numpy(eidx).to(dev)
    bt = torch.from_numpy(eidx // 128).to(dev)
    m = eidx.size
    q_in, s_in = [], []
    for qp, sp in zip(qs, ss):
        qq = np.zeros((m, 128), np.uint8)          # each sample is element 0 of its own block
        qq[:, 0] = _host(torch, qp[et])
        q_in.append(qq.ravel())
        s_in.append(_host(torch, sp[bt]))
    same(f32(_host(torch, y[et])), f32(oracle.dequant_reduce(q_in, s_in, fmt)[::128]),
         "dequant-reduce fp32 (sampled elements)")

    for j, (name, w) in enumerate(moe.items()):
        K = w.shape[-1]
        rows = w.numel() // K
        ridx = _sample_idx(rows, 512, seed=3 + j)
        rt = torch.from_numpy(ridx).to(dev)
        qm, em = oracle.mx8_quantize(_host(torch, w.view(rows, K)[rt]))
        same(_host(torch, mx_out[name][0].view(rows, K)[rt]), qm, "mx8 %s codes (sampled rows)" % name)
        same(_host(torch, mx_out[name][1][rt]), em, "mx8 %s e8m0 (sampled rows)" % name)
    covered.update({"sampled_quantize_blocks": int(idx.size), "sampled_reduce_elements": int(m),
                    "sampled_mx8_rows_per_tensor": 512})
    return covered


GATE_FRAC = 0.70                 # of the HBM peak, for every op at >= 64 MiB payloads


def gates(ops, side):
    """Pass / fail of every gated point: each op whose per-peer bf16
    payload is at least 64 MiB must reach GATE_FRAC of the HBM peak."""
    pts = []

    def add(name, frac):
        if frac is not None:
            pts.append({"point": name, "frac_peak": round(frac, 4), "pass": frac >= GATE_FRAC})

    add("quantize_e4m3 3.5e9 elements", ops["quantize_e4m3"]["frac_peak"])
    add("dequant_reduce_k8_f32 437.5M elements", ops["dequant_reduce_k8_f32"]["frac_peak"])
    add("mx8_layer 603,979,776 elements", ops["mx8_layer"]["frac_peak"])
    for row in side.get("payload_sweep_e5m2", []):
        if row["payload_bytes"] >= 64 << 20:
            add("payload_sweep quantize_e5m2 %d B" % row["payload_bytes"],
                row["quantize_hbm_GBps"] / HBM_PEAK_GBS)
            add("payload_sweep reduce_k8_f32 %d B" % row["payload_bytes"],
                row["reduce_k8_hbm_GBps"] / HBM_PEAK_GBS)
    for fmt_name, rec in side.get("stress_reduce_k8_bf16", {}).items():
        add("stress reduce_k8_bf16 full %s" % fmt_name, rec["full_frac_peak"])
    return {"threshold_frac_peak": GATE_FRAC, "points": pts,
            "all_pass": all(p["pass"] for p in pts)}


def device_info(torch, dev):
    """What the figures were measured on.  Clock and memory attributes come
    from hipDeviceGetAttribute in the HIP runtime this process already has
    loaded (found in its memory map; no second copy is ever loaded)."""
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2 ** 30, 1), "hip_runtime": torch.version.hip,
            "torch": torch.__version__}
    try:
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path:
            hip = ctypes.CDLL(path)
            attrs = {"peak_sclk_MHz": 5, "mem_bus_width_bits": 59, "peak_mclk_MHz": 60}
            for key, code in attrs.items():
                v = ctypes.c_int(0)
                if hip.hipDeviceGetAttribute(ctypes.byref(v), code, dev.index or 0) == 0:
                    info[key] = v.value // 1000 if key.endswith("MHz") else v.value
    except OSError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    return info


def median_ms(torch, fns):
    """Median HIP-event time of a list of launches (one event pair each)."""
    ts = []
    for fn in fns:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    v = sorted(a.elapsed_time(b) for a, b in ts)
    return v[len(v) // 2]


def graph_ms(torch, fns, replays=5, runs=3, all_runs=None):
    """Per-launch device time of back-to-back launches: the launches are
    captured once into a HIP graph (torch.cuda.CUDAGraph) and the graph is
    replayed, so host-side enqueue time never shows up between kernels.
    The graph is timed `runs` times (`replays` replays each, one event pair
    per run) and the median run is returned; the first run after a pause
    of the device measured up to 2% slower than the rest, and one run alone
    would carry that.  Every run's per-launch time goes to `all_runs` when a
    list is given."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(runs):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        b.synchronize()
        per.append(a.elapsed_time(b) / (replays * len(fns)))
    del g
    if all_runs is not None:
        all_runs.extend(per)
    return sorted(per)[len(per) // 2]


def host_latency_us(torch, fn, reps=50):
    """Host enqueue -> completion: median wall time of one call (argument
    checks, launch) followed by a device synchronize."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    ts.sort()
    return round(ts[len(ts) // 2] * 1e6, 1)


SWEEP_GRAPH_BYTES = 768e6   # bytes one sweep graph touches: 3x the Infinity Cache
SWEEP_MAX_LAUNCHES = 8192


def sweep_launches(bytes_per_launch, reps):
    """Launches per sweep graph: at least `reps`, and enough that one replay
    touches SWEEP_GRAPH_BYTES, so a window's bytes are long gone from the
    256 MB Infinity Cache when the next replay comes back to it."""
    need = int(SWEEP_GRAPH_BYTES // bytes_per_launch) + 1
    return max(reps, min(need, SWEEP_MAX_LAUNCHES))


def payload_sweep(torch, fq, workloads, dev, reps=20):
    """e5m2 block quantize and k = 8 fused reduce (fp32 out) at the payload
    sizes of the sweep, each launch on a different window of 2 GiB pools.
    Each graph holds at least `reps` launches, and at small payloads enough
    more (sweep_launches) that its windows total 768 MB, three times the
    256 MB Infinity Cache, so the timed bytes come from HBM at every size.
    Times are per launch of a graph of back-to-back launches; payloads up to
    4 MiB also get the host's enqueue-to-completion latency of one call."""
    n_pool = 1 << 30
    x = workloads.sweep_payload(2 * n_pool, seed=0, device=dev)
    q = torch.empty(n_pool, dtype=torch.uint8, device=dev)
    s = torch.empty(n_pool // 128, dtype=torch.float32, device=dev)
    fq.fp8q_quantize(x, fq.E5M2, q_out=q, scales_out=s)
    y = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    out = []
    for nbytes in workloads.SWEEP_BYTES:
        n = nbytes // 2
        span = (n_pool - 9 * n) // 128 * 128

        def off(i):
            return (i * 9 * n) % span // 128 * 128

        def quant(i):
            o = off(i)
            return lambda: fq.fp8q_quantize(x[o:o + n], fq.E5M2, q_out=q[o:o + n],
                                            scales_out=s[o // 128:o // 128 + fq.num_scales(n)])

        def red(i):
            o = off(i)
            qs = [q[o + p * n:o + (p + 1) * n] for p in range(8)]
            ss = [s[(o + p * n) // 128:(o + p * n) // 128 + fq.num_scales(n)] for p in range(8)]
            yo = (i * n) % ((1 << 28) - n) // 4 * 4
            return lambda: fq.fp8q_dequant_reduce(qs, ss, fq.E5M2, out=y[yo:yo + n])

        q_runs, r_runs = [], []
        nq = sweep_launches(QUANT_BYTES_PER_ELEM * n, reps)
        nr = sweep_launches(reduce_bytes_per_elem(8, 4) * n, reps)
        qm = graph_ms(torch, [quant(i) for i in range(nq)], all_runs=q_runs)
        rm = graph_ms(torch, [red(i) for i in range(nr)], all_runs=r_runs)
        row = {"payload_bytes": nbytes, "elements": n,
               "quantize_us": round(qm * 1e3, 2),
               "quantize_hbm_GBps": round(QUANT_BYTES_PER_ELEM * n / qm / 1e6, 1),
               "quantize_bf16_equiv_GBps": round(2 * n / qm / 1e6, 1),
               "reduce_k8_us": round(rm * 1e3, 2),
               "reduce_k8_hbm_GBps": round(reduce_bytes_per_elem(8, 4) * n / rm / 1e6, 1),
               "reduce_k8_bf16_equiv_GBps": round(16 * n / rm / 1e6, 1),
               "quantize_launches_per_graph": nq, "reduce_k8_launches_per_graph": nr,
               "quantize_us_runs": [round(v * 1e3, 2) for v in q_runs],
               "reduce_k8_us_runs": [round(v * 1e3, 2) for v in r_runs]}
        if nbytes <= 4 << 20:
            row["quantize_host_latency_us"] = host_latency_us(torch, quant(0))
            row["reduce_k8_host_latency_us"] = host_latency_us(torch, red(0))
        out.append(row)
    del x, q, s, y
    return out


def tiny_config(torch, fq, workloads, dev, reps=20):
    """The 1,048,576-element tiny gradient: e4m3 quantize, dequantize to fp32
    and the k = 4 reduce to fp32 (4 peers drawn with seeds 0-3).  At 2-8 MB
    the data stays in the 256 MB Infinity Cache, so these are cache-hot
    per-launch times in a graph of back-to-back launches, plus the host's
    enqueue-to-completion latency of one call."""
    xs = [workloads.tiny_gradient(p).to(dev) for p in range(4)]
    peers = [fq.fp8q_quantize(x, fq.E4M3) for x in xs]
    n = xs[0].numel()
    q0, s0 = peers[0]
    qo = torch.empty(n, dtype=torch.uint8, device=dev)
    so = torch.empty(fq.num_scales(n), dtype=torch.float32, device=dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    ops = {
        "quantize_e4m3": (lambda: fq.fp8q_quantize(xs[0], fq.E4M3, q_out=qo, scales_out=so),
                          QUANT_BYTES_PER_ELEM),
        "dequantize_f32": (lambda: fq.fp8q_dequantize(q0, s0, fq.E4M3, out=y),
                           reduce_bytes_per_elem(1, 4)),
        "reduce_k4_f32": (lambda: fq.fp8q_dequant_reduce([a for a, _ in peers],
                                                         [b for _, b in peers], fq.E4M3, out=y),
                          reduce_bytes_per_elem(4, 4)),
    }
    res = {"elements": n}
    for name, (fn, bpe) in ops.items():
        ms = graph_ms(torch, [fn] * reps)
        res[name] = {"us": round(ms * 1e3, 2), "GBps": round(bpe * n / ms / 1e6, 1),
                     "host_latency_us": host_latency_us(torch, fn)}
    return res


def next_rows(torch, fq, workloads, dev, x, qs, ss, moe, mx_out, reps=10):
    """The rows beyond the step, on the step's own data:
    - dequant-reduce -> requantize (e4m3 -> e4m3) of the 8 Pi0.5 shards;
    - MXFP8 dequantize of the MoE layer (bf16 out, as the receiver's weights)
      and an 8-peer MXFP8 reduce of gate-shaped expert tensors (fp32 out);
    - tensorwise e4m3 quantize of the 3.5e9-element gradient."""
    res = {}
    n = qs[0].numel()
    k = len(qs)
    q_o = torch.empty(n, dtype=torch.uint8, device=dev)
    s_o = torch.empty(fq.num_scales(n), dtype=torch.float32, device=dev)
    f = lambda: fq.fp8q_dequant_reduce_requantize(qs, ss, fq.E4M3, fq.E4M3, q_out=q_o, scales_out=s_o)
    f()
    ms = median_ms(torch, [f] * reps)
    alg = reduce_bytes_per_elem(k, 1 + 4 / 128) * n
    res["reduce_requantize_k8_e4m3"] = {"elements": n, "us": round(ms * 1e3, 2),
                                        "hbm_GBps": round(alg / ms / 1e6, 1),
                                        "frac_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del q_o, s_o

    ys = {name: torch.empty(w.shape, dtype=torch.bfloat16, device=dev) for name, w in moe.items()}

    def deq():
        for name in moe:
            fq.mx8_dequantize(mx_out[name][0], mx_out[name][1], out_dtype=torch.bfloat16,
                              out=ys[name])
    deq()
    ms = median_ms(torch, [deq] * reps)
    n_mx = sum(w.numel() for w in moe.values())
    alg = (1 + 1 / 32 + 2) * n_mx
    res["mx8_dequantize_layer_bf16"] = {"elements": n_mx, "us": round(ms * 1e3, 2),
                                        "hbm_GBps": round(alg / ms / 1e6, 1),
                                        "frac_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del ys
    shape = moe["gate"].shape
    peers = [fq.mx8_quantize(workloads.kaiming_uniform(shape, 100 + p, device=dev)) for p in range(8)]
    y = torch.empty(shape, dtype=torch.float32, device=dev)
    f = lambda: fq.mx8_dequant_reduce([a for a, _ in peers], [b for _, b in peers], out=y)
    f()
    ms = median_ms(torch, [f] * reps)
    nn = y.numel()
    alg = (8 * (1 + 1 / 32) + 4) * nn
    res["mx8_reduce_k8_f32"] = {"elements": nn, "us": round(ms * 1e3, 2),
                                "hbm_GBps": round(alg / ms / 1e6, 1),
                                "frac_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del peers, y

    nx = x.numel()
    q_t = torch.empty(nx, dtype=torch.uint8, device=dev)
    s_t = torch.empty(1, dtype=torch.float32, device=dev)
    f = lambda: fq.fp8q_quantize_tensorwise(x, fq.E4M3, q_out=q_t, scale_out=s_t)
    f()
    ms = median_ms(torch, [f] * reps)
    alg = 5.0 * nx
    res["quantize_tensorwise_e4m3"] = {"elements": nx, "us": round(ms * 1e3, 2),
                                       "hbm_GBps": round(alg / ms / 1e6, 1),
                                       "frac_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4),
                                       "bytes_per_element": 5}
    del q_t, s_t
    return res


def k_sweep(torch, fq, q, s, dev, reps=10, requantize=False):
    """Fused reduce into bf16 (or, with requantize, reduce -> e4m3 requantize)
    for k = 1, 2, 4, 8, 16 peers of 218,750,000 elements each, taken from 16
    distinct block-aligned slices of the quantized gradient.  Launch i reads
    slices (i * k + j) mod 16, so the inputs rotate through all 3.5 GB and
    come from HBM, not from the 256 MB Infinity Cache; the output alternates
    between two buffers.  Per-launch times are graph replays (graph_ms)."""
    n = q.numel() // 16
    stride = n // 128 * 128
    qs = [q[p * stride:p * stride + n] for p in range(16)]
    ss = [s[p * stride // 128:p * stride // 128 + fq.num_scales(n)] for p in range(16)]
    if requantize:
        outs = [(torch.empty(n, dtype=torch.uint8, device=dev),
                 torch.empty(fq.num_scales(n), dtype=torch.float32, device=dev)) for _ in range(2)]
        out_bytes = 1 + 4 / 128
    else:
        outs = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        out_bytes = 2
    out = []
    for k in (1, 2, 4, 8, 16):
        def launch(i, k=k):
            sel = [(i * k + j) % 16 for j in range(k)]
            qk, sk = [qs[p] for p in sel], [ss[p] for p in sel]
            if requantize:
                return lambda: fq.fp8q_dequant_reduce_requantize(
                    qk, sk, fq.E4M3, fq.E4M3, q_out=outs[i % 2][0], scales_out=outs[i % 2][1])
            return lambda: fq.fp8q_dequant_reduce(qk, sk, fq.E4M3, out_dtype=torch.bfloat16,
                                                  out=outs[i % 2])
        ms = graph_ms(torch, [launch(i) for i in range(reps)])
        alg = reduce_bytes_per_elem(k, out_bytes) * n
        out.append({"k": k, "elements": n, "us": round(ms * 1e3, 2),
                    "hbm_GBps": round(alg / ms / 1e6, 1),
                    "frac_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)})
    del outs
    return out


def stress_reduce(torch, fq, workloads, dev, reps=21):
    """k = 8 fused reduce into bf16 over the stress payload's shape: 8 peers x
    33,554,432 elements in 8 all-to-all chunks; "share" is one chunk (one
    GPU's part), "full" is all of it.  The reduce's time does not depend on
    the code values, so the shards are drawn directly as wire codes.  Seven
    copies of the 344 MB working set (2.4 GB) rotate from launch to launch so
    that the data comes from HBM, not from the 256 MB Infinity Cache."""
    n, chunks = workloads.STRESS_N, workloads.STRESS_CHUNKS
    copies = 7
    res = {}
    for fmt, name in ((fq.E4M3, "e4m3"), (fq.E5M2, "e5m2")):
        sets = []
        for c in range(copies):
            shards = [workloads.random_wire_shard(n, seed=300 + p, fmt=fmt, device=dev)
                      for p in range(8)]
            sets.append((shards, torch.empty(n, dtype=torch.bfloat16, device=dev)))
        cn = n // chunks

        def share(i):
            shards, y = sets[i % copies]
            j = (i // copies) % chunks
            qs = [a[j * cn:(j + 1) * cn] for a, _ in shards]
            ss = [b[j * cn // 128:(j + 1) * cn // 128] for _, b in shards]
            return lambda: fq.fp8q_dequant_reduce(qs, ss, fmt, out_dtype=torch.bfloat16,
                                                  out=y[j * cn:(j + 1) * cn])

        def full(i):
            shards, y = sets[i % copies]
            return lambda: fq.fp8q_dequant_reduce([a for a, _ in shards], [b for _, b in shards],
                                                  fmt, out_dtype=torch.bfloat16, out=y)
        f_runs = []
        sm = graph_ms(torch, [share(i) for i in range(reps)])
        fm = graph_ms(torch, [full(i) for i in range(reps)], all_runs=f_runs)
        alg = reduce_bytes_per_elem(8, 2)
        res[name] = {"share_elements": cn, "share_us": round(sm * 1e3, 2),
                     "share_hbm_GBps": round(alg * cn / sm / 1e6, 1),
                     "full_elements": n, "full_us": round(fm * 1e3, 2),
                     "full_hbm_GBps": round(alg * n / fm / 1e6, 1),
                     "full_frac_peak": round(alg * n / fm / 1e6 / HBM_PEAK_GBS, 4),
                     "full_us_runs": [round(v * 1e3, 2) for v in f_runs]}
        del sets
    return res


def mid_size_only(torch, fq, workloads, dev, reps):
    """The gated mid-size dispatches alone, each launched eagerly `reps`
    times on rotating inputs and timed with HIP events on the current
    stream (no HIP graphs, so that a profiler sees ordinary dispatches):
    the 64 MiB payload's e5m2 and e4m3 quantize and its k = 8 reduce into
    fp32, the full stress payload's k = 8 reduce into bf16 (e4m3, e5m2), and
    the k = 16 reduce into bf16 of 218,750,000-element peers.  Returns one
    record per op: mean, median and minimum launch time, and % of peak."""
    res = {}

    def timed(name, fns, alg_bytes):
        for f in fns[:2]:
            f()
        torch.cuda.synchronize()
        ev = []
        for f in fns:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        mean = sum(us) / len(us)
        res[name] = {"us": round(mean, 2), "us_median": round(us[len(us) // 2], 2),
                     "us_min": round(us[0], 2), "hbm_GBps": round(alg_bytes / mean / 1e3, 1),
                     "frac_peak": round(alg_bytes / mean / 1e3 / HBM_PEAK_GBS, 4)}

    # 64 MiB payload: windows of a 2 GiB bf16 pool, 8 peers for the reduce
    n_pool, n = 1 << 30, (64 << 20) // 2
    x = workloads.sweep_payload(2 * n_pool, seed=0, device=dev)
    q = torch.empty(n_pool, dtype=torch.uint8, device=dev)
    s = torch.empty(n_pool // 128, dtype=torch.float32, device=dev)
    fq.fp8q_quantize(x, fq.E5M2, q_out=q, scales_out=s)
    y = torch.empty(4 * n, dtype=torch.float32, device=dev)
    win = [(i * 9 * n) % (n_pool - 9 * n) // 128 * 128 for i in range(reps)]
    for fmt, name in ((fq.E5M2, "quantize_e5m2_64MiB"), (fq.E4M3, "quantize_e4m3_64MiB")):
        timed(name, [lambda o=o, fmt=fmt: fq.fp8q_quantize(
            x[o:o + n], fmt, q_out=q[o:o + n], scales_out=s[o // 128:o // 128 + n // 128])
            for o in win], QUANT_BYTES_PER_ELEM * n)
    fq.fp8q_quantize(x, fq.E5M2, q_out=q, scales_out=s)
    timed("reduce_k8_f32_64MiB", [lambda o=o, i=i: fq.fp8q_dequant_reduce(
        [q[o + p * n:o + (p + 1) * n] for p in range(8)],
        [s[(o + p * n) // 128:(o + (p + 1) * n) // 128] for p in range(8)], fq.E5M2,
        out=y[(i % 4) * n:(i % 4 + 1) * n]) for i, o in enumerate(win)],
        reduce_bytes_per_elem(8, 4) * n)
    del x, q, s, y
    # the stress payload's full k = 8 reduce into bf16, 7 copies rotating
    ns = workloads.STRESS_N
    for fmt, name in ((fq.E4M3, "stress_reduce_k8_bf16_e4m3"), (fq.E5M2, "stress_reduce_k8_bf16_e5m2")):
        sets = [([workloads.random_wire_shard(ns, seed=300 + p, fmt=fmt, device=dev)
                  for p in range(8)], torch.empty(ns, dtype=torch.bfloat16, device=dev))
                for _ in range(7)]
        timed(name, [lambda c=sets[i % 7], fmt=fmt: fq.fp8q_dequant_reduce(
            [a for a, _ in c[0]], [b for _, b in c[0]], fmt, out_dtype=torch.bfloat16, out=c[1])
            for i in range(reps)], reduce_bytes_per_elem(8, 2) * ns)
        del sets
    # k = 16 into bf16: 16 peers of 218,750,000 elements, two output buffers
    nk = 218_750_000
    peers = [workloads.random_wire_shard(nk, seed=400 + p, fmt=fq.E4M3, device=dev) for p in range(16)]
    outs = [torch.empty(nk, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    timed("reduce_k16_bf16_218.75M", [lambda i=i: fq.fp8q_dequant_reduce(
        [a for a, _ in peers], [b for _, b in peers], fq.E4M3, out_dtype=torch.bfloat16,
        out=outs[i % 2]) for i in range(reps)], reduce_bytes_per_elem(16, 2) * nk)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-frac", type=float, default=1 / 8,
                    help="fraction of the workload the CPU oracle baseline runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true", help="skip the naive-path side figures")
    ap.add_argument("--copy-reference-gib", type=float, default=1.0,
                    help="size of the plain device copy run once for counter calibration")
    ap.add_argument("--mid-size-only", action="store_true",
                    help="run only the gated mid-size dispatches, eagerly (for profiling); "
                         "prints their timings as one JSON line")
    args = ap.parse_args()

    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU: the library has no multi-GPU path "
                         "(got --gpus %d). Run with --gpus 1.\n" % args.gpus)
        sys.exit(2)

    import torch

    import dequantize_reduce_transfer_amd as fq
    from dequantize_reduce_transfer_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mid_size_only:
        if args.copy_reference_gib > 0:
            nb = int(args.copy_reference_gib * (1 << 30))
            src = torch.empty(nb, dtype=torch.uint8, device=dev)
            src.fill_(1)
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
            del src
        log("mid-size dispatches, %d launches each" % args.steps)
        print(json.dumps({"mid_size_only": True, "steps": args.steps,
                          "ops": mid_size_only(torch, fq, workloads, dev, args.steps),
                          "env": device_info(torch, dev)}), flush=True)
        return
    fmt = fq.E4M3
    n = workloads.PI05_N
    k = workloads.PI05_PEERS
    n_shard = workloads.PI05_SHARD_N

    log("generating the %.2e-element bf16 gradient on the GPU" % n)
    x = workloads.segmented_gradient(n, seed=0, device=dev)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    s = torch.empty(fq.num_scales(n), dtype=torch.float32, device=dev)

    log("quantizing once; the %d peer shards are block-aligned slices of the codes" % k)
    fq.fp8q_quantize(x, fmt, q_out=q, scales_out=s)
    stride = n_shard // 128 * 128
    qs = [q[p * stride:p * stride + n_shard] for p in range(k)]
    ss = [s[p * stride // 128:p * stride // 128 + fq.num_scales(n_shard)] for p in range(k)]
    peers = list(zip(qs, ss))
    y = torch.empty(n_shard, dtype=torch.float32, device=dev)

    log("generating the MoE layer")
    moe = workloads.moe_layer(seed=0, device=dev)
    mx_out = {name: (torch.empty(w.shape, dtype=torch.uint8, device=dev),
                     torch.empty((w.numel() // w.shape[-1], w.shape[-1] // 32),
                                 dtype=torch.uint8, device=dev)) for name, w in moe.items()}
    n_mx = sum(w.numel() for w in moe.values())

    # one plain device copy of known size, for calibrating HBM byte counters
    if args.copy_reference_gib > 0:
        nb = int(args.copy_reference_gib * (1 << 30))
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    timer = Timer(torch)

    def step():
        timer.run("quantize", lambda: fq.fp8q_quantize(x, fmt, q_out=q, scales_out=s))
        timer.run("dequant_reduce", lambda: fq.fp8q_dequant_reduce(qs, ss, fmt, out=y))
        for name, w in moe.items():
            qo, eo = mx_out[name]
            timer.run("mx8_" + name, lambda w=w, qo=qo, eo=eo: fq.mx8_quantize(w, q_out=qo, e8m0_out=eo))

    log("warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.reset()

    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps

    bf16_bytes_step = 2 * n + 2 * k * n_shard + 2 * n_mx
    value = bf16_bytes_step / (elapsed / args.steps) / 1e9

    ops = {}
    q_ms = timer.mean_ms("quantize")
    r_ms = timer.mean_ms("dequant_reduce")
    q_alg = QUANT_BYTES_PER_ELEM * n
    r_alg = reduce_bytes_per_elem(k, 4) * n_shard
    ops["quantize_e4m3"] = {"elements": n, "us": round(q_ms * 1e3, 2),
                            "bf16_equiv_GBps": round(2 * n / q_ms / 1e6, 1),
                            "hbm_GBps": round(q_alg / q_ms / 1e6, 1),
                            "frac_peak": round(q_alg / q_ms / 1e6 / HBM_PEAK_GBS, 4),
                            **timer.spread_us("quantize")}
    ops["dequant_reduce_k8_f32"] = {"elements": n_shard, "us": round(r_ms * 1e3, 2),
                                    "bf16_equiv_GBps": round(2 * k * n_shard / r_ms / 1e6, 1),
                                    "hbm_GBps": round(r_alg / r_ms / 1e6, 1),
                                    "frac_peak": round(r_alg / r_ms / 1e6 / HBM_PEAK_GBS, 4),
                                    **timer.spread_us("dequant_reduce")}
    mx_ms = 0.0
    for name, w in moe.items():
        ms = timer.mean_ms("mx8_" + name)
        mx_ms += ms
        alg = MX_BYTES_PER_ELEM * w.numel()
        ops["mx8_" + name] = {"elements": w.numel(), "us": round(ms * 1e3, 2),
                              "hbm_GBps": round(alg / ms / 1e6, 1),
                              "frac_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4),
                              **timer.spread_us("mx8_" + name)}
    ops["mx8_layer"] = {"elements": n_mx, "us": round(mx_ms * 1e3, 2),
                        "hbm_GBps": round(MX_BYTES_PER_ELEM * n_mx / mx_ms / 1e6, 1),
                        "frac_peak": round(MX_BYTES_PER_ELEM * n_mx / mx_ms / 1e6 / HBM_PEAK_GBS, 4)}

    side = {}
    if not args.no_side:
        log("side figures: dequantize alone and the naive dequantize-then-sum")
        parts = [torch.empty(n_shard, dtype=torch.float32, device=dev) for _ in range(k)]
        t2 = Timer(torch)
        for it in range(3 + 10):
            if it == 3:
                torch.cuda.synchronize()
                t2.reset()
            for p in range(k):
                t2.run("dequantize", lambda p=p: fq.fp8q_dequantize(qs[p], ss[p], fmt, out=parts[p]))
            t2.run("sum", lambda: fq.fp8q_sum_f32(parts, out=y))
        torch.cuda.synchronize()
        d_ms = t2.mean_ms("dequantize")
        naive_ms = k * d_ms + t2.mean_ms("sum")
        d_alg = reduce_bytes_per_elem(1, 4) * n_shard
        side["dequantize_f32"] = {"elements": n_shard, "us": round(d_ms * 1e3, 2),
                                  "hbm_GBps": round(d_alg / d_ms / 1e6, 1),
                                  "frac_peak": round(d_alg / d_ms / 1e6 / HBM_PEAK_GBS, 4)}
        side["naive_dequant_then_sum_k8_us"] = round(naive_ms * 1e3, 2)
        side["fused_speedup_vs_naive"] = round(naive_ms / r_ms, 2)
        log("side figures: the step captured in a HIP graph")

        def plain_step():
            fq.fp8q_quantize(x, fmt, q_out=q, scales_out=s)
            fq.fp8q_dequant_reduce(qs, ss, fmt, out=y)
            for name, w in moe.items():
                fq.mx8_quantize(w, q_out=mx_out[name][0], e8m0_out=mx_out[name][1])
        g_ms = graph_ms(torch, [plain_step], replays=10)
        side["step_in_hip_graph"] = {"ms_per_step": round(g_ms, 4),
                                     "bf16_equiv_GBps": round(bf16_bytes_step / g_ms / 1e6, 1),
                                     "eager_ms_per_step": round(ms_step, 4)}
        del parts
        log("side figures: requantize, MXFP8 receiver, tensorwise")
        side.update(next_rows(torch, fq, workloads, dev, x, qs, ss, moe, mx_out))
        log("side figures: peer-count sweep")
        side["reduce_k_sweep_bf16"] = k_sweep(torch, fq, q, s, dev)
        side["requantize_k_sweep_e4m3"] = k_sweep(torch, fq, q, s, dev, requantize=True)
        log("side figures: tiny gradient (cache-resident)")
        side["tiny_gradient"] = tiny_config(torch, fq, workloads, dev)
        log("side figures: payload sweep (e5m2) and stress reduce (bf16 out)")
        side["payload_sweep_e5m2"] = payload_sweep(torch, fq, workloads, dev)
        side["stress_reduce_k8_bf16"] = stress_reduce(torch, fq, workloads, dev)

    roofline = {
        "bound": "hbm",
        "kernel": "quantize_kernel<E4M3> (block-128 quantize, 3.5e9 elements)",
        "achieved": round(q_alg / q_ms / 1e6, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(q_alg / q_ms / 1e6 / HBM_PEAK_GBS, 4),
        "traffic": read_traffic(QUANT_KERNEL_SRCS),
        "algorithmic_bytes_per_launch": q_alg,
        "avg_launch_us": round(q_ms * 1e3, 2),
    }

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "pi05_gradient_fp8_wire_step",
            "quantize": "block-128 e4m3, 3,500,000,000 bf16 elements (segments of 25M, "
                        "std log-uniform 1e-6..1e-2)",
            "dequant_reduce": "k=8 peer shards x 437,500,000 elements -> fp32 (block-aligned "
                              "slices of the quantized gradient)",
            "mx8": "Qwen3-30B-A3B MoE layer, 128 experts, gate/up [768,2048], down [2048,768]",
            "bf16_equiv_bytes_per_step": bf16_bytes_step,
        },
        "roofline": roofline,
        "ops": ops,
        "side": side,
        "env": device_info(torch, dev),
    }

    out["gates"] = gates(ops, side)

    parity_error = None
    out["parity_checked"] = False
    if not args.no_cpu_baseline:
        smp = _cpu_sample(x, peers, moe, args.cpu_frac)
        smp["frac"] = args.cpu_frac
        threads = host_threads()
        log("CPU baseline: oracle on %.4g of the workload, %d threads" % (args.cpu_frac, threads))
        rec, outputs = cpu_baseline(smp, fmt, threads, runs=3 if threads > 1 else 1)
        rec.update(host_cpus())
        rec["thread_cap"] = HOST_THREAD_CAP
        rec["thread_cap_reason"] = ("the host's CPU share for one GPU; the pool "
                                    "uses min(cap, affinity_cpus) threads")
        out["cpu_baseline"] = rec
        log("parity: the step's outputs against the oracle")
        try:
            out["parity"] = step_parity(torch, fmt, smp, outputs, x, q, s, qs, ss, y, moe, mx_out)
            out["parity_checked"] = True
        except AssertionError as e:
            parity_error = str(e)
            out["parity"] = {"mismatch": parity_error}
        del outputs
        if threads > 1:
            log("CPU baseline: the same sample on one thread")
            side["cpu_baseline_1_thread"] = cpu_baseline(smp, fmt, 1)[0]
        del smp
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)
    if parity_error is not None:
        log("PARITY FAILURE: " + parity_error)
        sys.exit(3)


if __name__ == "__main__":
    main()
