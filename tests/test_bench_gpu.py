"""bench.py end to end on the GPU (short runs): the stdout line the driver
parses carries every field of the benchmark contract, stays short, and the
profiler mode and the counter calibration run."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*extra, timeout=300):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *extra], capture_output=True, text=True,
                       timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.strip().splitlines() if l.strip()]
    return lines, r.stderr


def test_bench_driver_shape_with_one_point_sweep():
    """The driver's argument shape (--gpus 1 --steps --warmup) with a
    one-point sweep: one stdout line under 4 KB, with the roofline and the
    CPU baseline filled in."""
    lines, err = _bench("--gpus", "1", "--steps", "3", "--warmup", "1", "--M", "1", "--sweep-workloads", "1",
                        "--sweep-reps", "5", "--cpu-budget", "1")
    assert len(lines) == 1, lines[-3:]
    assert len(lines[0].encode()) < 4096, len(lines[0])
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline",
              "stream_ordered", "stream_ordered_best", "stream_ordered_graph", "policy_graph", "sweep",
              "sweep_columns"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["unit"] == "TFLOP/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "gpt3_175b_mlp_tp8_f16" and d["config"]["M"] == 1
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s" and 0 < roof["frac"] < 1
    assert roof["achieved"] == pytest.approx(roof["frac"] * roof["peak"], rel=1e-3)
    cpu = d["cpu_baseline"]
    assert cpu is not None and cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["cpu_model"] and cpu["nproc"] >= 1
    for k in ("stream_ordered", "stream_ordered_best", "stream_ordered_graph"):
        assert d[k]["value"] > 0 and d[k]["plan"][1] >= 1
    assert d["policy_graph"]["value"] > 0 and d["policy_graph"]["ms_per_step"] > 0
    assert len(d["sweep"]) == 1 and len(d["sweep"][0]) == len(d["sweep_columns"])
    rows = [json.loads(l) for l in err.splitlines() if l.startswith("{")]
    assert sorted(r["policy"] for r in rows) == ["row_sync", "stream_ordered", "tile_sync"]


def test_bench_kernels_only_and_copy_calibration():
    lines, _ = _bench("--steps", "2", "--warmup", "1", "--kernels-only")
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["config"]["M"] == 2048 and d["roofline"]["bound"] == "mfma" and d["value"] > 0
    assert d["cpu_baseline"] is None and "sweep" not in d
    lines, err = _bench("--copy-mib", "64")
    assert lines == [] and "copied 64 MiB x 3" in err
