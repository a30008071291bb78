"""bench.py end to end on a small workload: one JSON line with the fields the
measurement promises (run as a child process, as the bench is run on its own)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_complete_json_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "sq4096", "--steps", "2",
           "--warmup", "1", "--no-cpu-baseline"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "step_ms", "kernels",
                "probe_peaks"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 2 and r["warmup"] == 1
    assert r["value"] > 0 and r["ms_per_step"] > 0
    assert r["config"]["visible_pairs"] == 4 * 1024 * 1025 // 2  # sum over t < 4096 of t // 4 + 1
    rl = r["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2500.0
    assert 0.0 < rl["frac"] < 1.0 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-9
    assert r["step_ms"]["min"] <= r["step_ms"]["median"] <= r["step_ms"]["max"]
    assert r["probe_peaks"]["hbm_copy_GBs"] > 0 and r["probe_peaks"]["bf16_gemm_TFLOPs"] > 0
    c = r["config"]
    assert c["chunk_buffers"] in (1, 2) and c["workspace_bytes"] > 0 and c["pooling"] == "mean"
    assert c["score_bytes_in_flight"] == c["chunk_buffers"] * c["score_bytes_per_chunk_buffer"]
    tk = r["kernels"]["topk"]
    assert tk["frac"] is None or 0.0 < tk["frac"] <= 1.0       # counter bytes, never above the peak
    assert tk["frac_if_every_score_were_read"] > 0


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
