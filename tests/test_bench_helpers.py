"""Host logic of the benchmark (no GPU): the counter-summary guard and the
block-aligned pieces of the CPU baseline."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_source_digest_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n/* block */\n")
    b.write_text("int f(int x) { return x + 1; }\n// a different comment\n")
    assert bench.source_digest([str(a)]) == bench.source_digest([str(b)])
    b.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest([str(a)]) != bench.source_digest([str(b)])


def test_read_traffic_refuses_a_changed_kernel(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    assert bench.read_traffic([str(src)]) is None


@pytest.mark.parametrize("total,parts,multiple", [(1, 1, 128), (127, 4, 128), (437_499_904, 64, 128),
                                                  (5_000, 64, 1), (128 * 1000 + 77, 7, 128)])
def test_cpu_pieces_tile_the_range(total, parts, multiple):
    step = bench._piece(total, parts, multiple)
    assert step % multiple == 0 and step >= multiple
    starts = list(range(0, total, step))
    assert len(starts) <= max(parts, 1) + 1
    assert all(s % multiple == 0 for s in starts)
    assert min(total, starts[-1] + step) == total


@pytest.mark.parametrize("nbytes", [65536, 262144, 785408, 4194304, 16777216, 67108864])
def test_sweep_graphs_span_three_infinity_caches(nbytes):
    """Each payload-sweep graph touches at least 768 MB (three times the
    256 MB Infinity Cache) and holds at least the 20 launches asked for, up
    to the launch cap, for the quantize and for the k = 8 reduce."""
    n = nbytes // 2
    for per_elem in (bench.QUANT_BYTES_PER_ELEM, bench.reduce_bytes_per_elem(8, 4)):
        m = bench.sweep_launches(per_elem * n, 20)
        assert m >= 20 and m <= max(20, bench.SWEEP_MAX_LAUNCHES)
        assert m * per_elem * n >= bench.SWEEP_GRAPH_BYTES or m == bench.SWEEP_MAX_LAUNCHES
    assert bench.sweep_launches(bench.QUANT_BYTES_PER_ELEM * 32768, 20) == 7732
    assert bench.sweep_launches(bench.QUANT_BYTES_PER_ELEM * (1 << 25), 20) == 20


def test_gates_flag_every_gated_point():
    ops = {"quantize_e4m3": {"frac_peak": 0.84}, "dequant_reduce_k8_f32": {"frac_peak": 0.80},
           "mx8_layer": {"frac_peak": 0.79}}
    side = {"payload_sweep_e5m2": [
                {"payload_bytes": 16 << 20, "quantize_hbm_GBps": 3000.0, "reduce_k8_hbm_GBps": 5000.0},
                {"payload_bytes": 64 << 20, "quantize_hbm_GBps": 5560.0, "reduce_k8_hbm_GBps": 6100.0}],
            "stress_reduce_k8_bf16": {"e4m3": {"full_frac_peak": 0.75},
                                      "e5m2": {"full_frac_peak": 0.71}}}
    g = bench.gates(ops, side)
    names = [p["point"] for p in g["points"]]
    assert len(names) == 7 and not any("16777216" in s for s in names)
    by = {p["point"]: p["pass"] for p in g["points"]}
    assert by["payload_sweep quantize_e5m2 67108864 B"] is False      # 69.5%
    assert by["payload_sweep reduce_k8_f32 67108864 B"] is True
    assert g["all_pass"] is False
    side["payload_sweep_e5m2"][1]["quantize_hbm_GBps"] = 5600.0
    assert bench.gates(ops, side)["all_pass"] is True


def test_host_cpus_and_thread_cap():
    h = bench.host_cpus()
    assert h["os_cpu_count"] == os.cpu_count()
    assert 1 <= h["affinity_cpus"] <= os.cpu_count()
    assert 1 <= bench.host_threads() <= bench.HOST_THREAD_CAP


def _cpu_step(n_q=128 * 777 + 128, n_r=128 * 301):
    """A small stand-in for the step's tensors, made by the oracle on the CPU
    in place of the GPU (x, q, s, peers, y, MoE weights and their codes)."""
    import numpy as np
    import torch

    import oracle
    from dequantize_reduce_transfer_amd import workloads

    x = workloads.tiny_gradient(0, n=n_q, zero_block=3)
    qa, sa = oracle.quantize(workloads.bits(x), 0)
    q, s = torch.from_numpy(qa), torch.from_numpy(sa)
    stride = n_r // 2 // 128 * 128
    qs = [q[p * stride:p * stride + n_r] for p in range(2)]
    ss = [s[p * stride // 128:p * stride // 128 + (n_r + 127) // 128] for p in range(2)]
    y = torch.from_numpy(oracle.dequant_reduce([a.numpy() for a in qs], [b.numpy() for b in ss], 0))
    moe = {"gate": workloads.kaiming_uniform((4, 8, 64), 0), "down": workloads.kaiming_uniform((4, 16, 32), 1)}
    mx = {}
    for name, w in moe.items():
        qm, em = oracle.mx8_quantize(workloads.bits(w))
        mx[name] = (torch.from_numpy(qm), torch.from_numpy(em))
    return x, q, s, qs, ss, y, moe, mx, np


@pytest.mark.parametrize("threads", [1, 3])
def test_cpu_baseline_outputs_reassemble_and_step_parity(threads, monkeypatch):
    import torch

    x, q, s, qs, ss, y, moe, mx, np = _cpu_step()
    smp = bench._cpu_sample(x, list(zip(qs, ss)), moe, 0.5)
    smp["frac"] = 0.5
    rec, outs = bench.cpu_baseline(smp, 0, threads)
    assert rec["cores"] == threads and rec["kind"] == "oracle" and rec["value"] > 0
    got = bench.step_parity(torch, 0, smp, outs, x, q, s, qs, ss, y, moe, mx)
    assert got["quantize_elements"] == smp["n_q"] and got["reduce_elements"] == smp["n_r"]
    # one flipped code inside the sample, then one outside it, are both caught
    for pos in (5, q.numel() - 3):
        q2 = q.clone()
        q2[pos] ^= 1
        with pytest.raises(AssertionError, match="quantize codes"):
            bench.step_parity(torch, 0, smp, outs, x, q2, s, qs, ss, y, moe, mx)
    y2 = y.clone()
    y2[-1] = y2[-1] * 2 + 1
    with pytest.raises(AssertionError, match="dequant-reduce"):
        bench.step_parity(torch, 0, smp, outs, x, q, s, qs, ss, y2, moe, mx)
    mx2 = dict(mx)
    e2 = mx["down"][1].clone()
    e2[-1, -1] ^= 1
    mx2["down"] = (mx["down"][0], e2)
    with pytest.raises(AssertionError, match="mx8 down e8m0"):
        bench.step_parity(torch, 0, smp, outs, x, q, s, qs, ss, y, moe, mx2)
