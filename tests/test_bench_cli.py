"""bench.py's command-line contract: one GPU only, and one JSON line with the
fields the measurement needs (the latter on a GPU)."""

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
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    print("CASE bench.py --steps 2 --warmup 1 --no-video --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1", "--no-video", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert "traffic" in rf and "achieved" in rf
    assert "workload" in d["config"]


@pytest.mark.gpu
def test_share_runs_small():
    """bench.share_runs on a small tensor (8 heads, 1024 tokens over 8
    GPUs): one head per GPU for Ulysses, 128 query rows per ring rank."""
    import torch
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    print("CASE bench.share_runs B=1 H=8 N=1024 D=128", flush=True)
    q, k, v = workloads.make_qkv(7, 1, 8, 1024, 1024, 128, device="cuda")
    s = bench.share_runs(q, k, v, 128 ** -0.5, reps=2, n_gpus=8)
    assert s["n_gpus"] == 8 and s["flop_per_gpu"] == 4.0 * 8 * 1024 * 1024 * 128 / 8
    u, r = s["ulysses_8"], s["ring_8"]
    assert u["shape"] == "B=1, H=1 of 8, N=1024, D=128"
    assert u["attn_fwd"]["reps"] == 2 and u["attn_fwd"]["median_ms"] > 0
    assert u["seq_concat_qkv_ms_median"] > 0 and u["seq_split_o_ms_median"] > 0
    assert u["layout_bytes"] == 2 * 4 * 1 * 1024 * 128 * 2
    assert r["reps"] == 2 and r["median_ms"] > 0 and r["accum_step_ms_median"] > 0
    assert 0 < r["frac_bf16_peak"] < 1 and 0 < u["attn_fwd"]["frac_bf16_peak"] < 1
