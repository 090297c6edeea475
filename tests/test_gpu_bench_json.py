"""bench.py's output contract on the GPU: one JSON line on stdout with the required
keys, the roofline object and the graph-replay statistics, from a short run on the
tiny workload (no CPU baseline, no extra workloads)."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract_keys():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print("case bench tiny_stacked", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_stacked", "--steps", "5",
                        "--warmup", "1", "--ramp", "0.1", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(d[key], kind), key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("tiny_stacked")
    roof = d["roofline"]
    assert roof["bound"] in ("mfma", "hbm") and roof["unit"] in ("TFLOP/s", "GB/s")
    assert roof["peak"] in (5000.0, 8000.0) and 0 < roof["achieved"]
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    g = d["config"]["graph_replay"]
    assert g["replays"] == 7 and g["calls_per_graph"] >= 1
    assert 0 < g["us_min"] <= g["us_per_call"] and g["us_iqr"] >= 0 and g["t_star_over_t"] > 0
