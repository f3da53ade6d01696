"""bench.py end to end on the GPU (short run): one JSON line with the
fields the benchmark contract requires and sane values."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-sweep", "--no-cpu"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.strip().splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline",
              "stream_ordered", "stream_ordered_best", "stream_ordered_graph"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["unit"] == "TFLOP/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "gpt3_175b_mlp_tp8_f16" and d["config"]["M"] == 2048
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["peak"] == 2500.0 and 0 < roof["frac"] < 1
    assert roof["achieved"] == pytest.approx(roof["frac"] * roof["peak"], rel=1e-3)
    for k in ("stream_ordered", "stream_ordered_best", "stream_ordered_graph"):
        assert d[k]["value"] > 0 and d[k]["plan"]["S1"] >= 1
