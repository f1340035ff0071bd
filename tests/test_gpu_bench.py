"""bench.py's JSON line on a GPU: a short run must keep the contract (one
line, the metric and units, the roofline and CPU-oracle objects, and a value
consistent with its own step time and byte count)."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("mode,extra,rows", [
    ("full", [], 1024), ("shard", [], 128),
    ("full", ["--tokens", "300", "--partials", "3", "--no-split"], 300),
    ("full", ["--workload", "tiny"], 64)])
def test_bench_line_keeps_the_contract(mode, extra, rows):
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    print(f"[case] bench.py --mode {mode} --steps 40 --warmup 10 {' '.join(extra)}", flush=True)
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--mode", mode,
                          "--steps", "40", "--warmup", "10", "--cpu-seconds", "0.5",
                          "--no-unfused", *extra], capture_output=True, text=True, timeout=240)
    assert run.returncode == 0, run.stderr[-2000:]
    lines = [ln for ln in run.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "settle"):
        assert key in d, key
    assert d["settle"]["steps"] >= 50 and d["settle"]["seconds"] > 0
    assert d["unit"] == "GB/s" and d["n_gpus"] == 1 and d["steps"] == 40 and d["warmup"] == 10
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    cfg = d["config"]
    assert cfg["rows"] == rows
    if "--tokens" in extra:
        assert cfg["num_tokens"] == 300 and cfg["num_partials"] == 3
        assert d["roofline"]["traffic"] is None    # counters belong to the default shape only
    itemsize = 2 if cfg["storage_dtype"] == "bf16" else 4
    assert f"{cfg['storage_dtype']} storage" in cfg["workload"]
    step_bytes = (cfg["num_partials"] + 3) * rows * cfg["hidden"] * itemsize
    assert abs(d["value"] - step_bytes / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - d["value"] / 8000.0) < 1e-3
    assert 0 < r["frac"] < 1
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] == 1 and c["value"] > 0
