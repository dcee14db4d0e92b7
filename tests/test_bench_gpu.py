"""The benchmark's output line on a GPU: one JSON object with the fields and
units its readers rely on, from a short run (few steps, small CPU budget)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_json_line():
    print("bench json line", flush=True)
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20", "--warmup", "200",
                           "--no-extra", "--cpu-budget", "1.5"], capture_output=True, text=True, timeout=600,
                          cwd=ROOT)
    assert proc.returncode == 0, proc.stderr[-2000:]
    lines = [l for l in proc.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, proc.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 200
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["vs_baseline"] is None
    assert d["config"]["workload"] == "ffn_gate_up_down_m1"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is the fused step's own algorithmic bytes over its time: the gate|up
    # launch (x in, fp16 h out) and the down GEMV on h
    step_bytes = 25_296_896 + 12_640_256
    assert d["config"]["bytes_per_step"] == step_bytes
    assert abs(d["value"] - step_bytes / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    # the same linears as three plain GEMVs, beside it
    plain = d["config"]["plain_three_gemv"]
    assert plain["bytes_per_step"] == 12_689_408 * 2 + 12_640_256
    assert abs(plain["GBs"] - plain["bytes_per_step"] / (plain["us_per_step"] * 1e-6) / 1e9) <= 0.01 * plain["GBs"]
    # the untimed work is stated
    assert d["settle_steps"] > 0 and str(d["settle_steps"]) in d["config"]["untimed"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["achieved"] < r["peak"]
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 25_296_896
    assert r["traffic_note"].startswith("stored") == (r["traffic"] is not None)
    # the loads alone of the same packed bytes, one launch each
    assert 0 < r["read_ceiling_us"] and 0 < r["frac_of_read_ceiling"] < 1.5
    assert d["extra"]["stream_read_us"]["gate_12.6MB"] > 0
    # each linear against the HBM peak, and its time at 75 % of it
    ex = d["extra"]
    assert set(ex["frac_of_peak_per_launch"]) == set(ex["GBs_per_launch"]) >= {"gate", "up", "down"}
    for p, f in ex["frac_of_peak_per_launch"].items():
        assert abs(f - ex["GBs_per_launch"][p] / 8000.0) < 1e-3
    assert ex["us_at_75pct_of_peak"]["gate"] == 2.115 and ex["us_at_75pct_of_peak"]["down"] == 2.107
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "GB/s" and c["value"] > 0
    assert c["cores"] == len(os.sched_getaffinity(0))  # the CPUs this process may use
    assert 1 <= c["blas_threads"] <= c["cores"]
    assert c["unpack_s"] > 0 and c["matvec_s"] > 0
    assert abs(c["unpack_s"] + c["matvec_s"] - c["pass_s"]) <= 1e-4
    assert isinstance(c["sample"], str) and c["sample"]
