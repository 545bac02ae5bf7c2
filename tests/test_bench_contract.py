"""The benchmark's command-line contract: more than one GPU is refused with a
message (no GPU needed), and a short GPU run prints exactly one JSON line
with every field the contract names, its gate flags, and the result of
checking the step's own outputs against the oracle."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_short_run_prints_one_contract_line():
    from gpu_util import require_gpu
    require_gpu()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1", "--no-side", "--cpu-frac", "0.004"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "gates", "parity_checked"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"] and "model" not in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # the step's own outputs were checked against the oracle
    assert d["parity_checked"] is True and d["parity"]["quantize_elements"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == min(cb["thread_cap"], cb["affinity_cpus"])
    assert cb["os_cpu_count"] >= cb["affinity_cpus"] >= 1 and "cpu_model" in cb
    assert {p["point"].split()[0] for p in d["gates"]["points"]} >= {
        "quantize_e4m3", "dequant_reduce_k8_f32", "mx8_layer"}


@pytest.mark.gpu
def test_mid_size_only_prints_every_gated_dispatch():
    """bench.py --mid-size-only (the profiling run of the gated mid-size
    dispatches) prints one JSON line with a timing for each of them."""
    from gpu_util import require_gpu
    require_gpu()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--mid-size-only",
                        "--steps", "3", "--copy-reference-gib", "0"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["mid_size_only"] is True and d["steps"] == 3
    assert set(d["ops"]) == {"quantize_e5m2_64MiB", "quantize_e4m3_64MiB", "reduce_k8_f32_64MiB",
                             "stress_reduce_k8_bf16_e4m3", "stress_reduce_k8_bf16_e5m2",
                             "reduce_k16_bf16_218.75M"}
    for rec in d["ops"].values():
        assert 0 < rec["us_min"] <= rec["us_median"] and 0 < rec["frac_peak"] < 1
