"""Host-side logic of bench.py (no GPU): the roofline bound and time, the
traffic summary lookup (used only for the sources and plan it was measured
on), the stream-ordered search space, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench
from consumer_gemm_chain_amd import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofline_bound_switches_near_the_ridge():
    w = gen.WORKLOADS[1]                               # GPT-3 shard, fp16
    for M, bound in ((1, "hbm"), (64, "hbm"), (256, "hbm"), (512, "mfma"), (2048, "mfma")):
        t, b = bench.roofline_time_us(w, M, w.dtype)
        assert b == bound, (M, b)
        f, by = w.flops(M), w.bytes(M)
        assert t == pytest.approx(max(f / 2.5e15, by / 8e12) * 1e6)
    # M = 2048: 618.5 GFLOP at 2.5 PFLOP/s
    assert bench.roofline_time_us(w, 2048, w.dtype)[0] == pytest.approx(247.39, abs=0.01)


def _summary(tmp_path, sources, plan, value=123456789):
    d = tmp_path / "profiles"
    d.mkdir(exist_ok=True)
    (d / "k_wl_M8_traffic.md").write_text(f"# summary\n\nsources: {sources}\nplan: {plan}\n"
                                          f"traffic_bytes_per_launch: {value}\n")
    return d


def test_traffic_summary_is_used_only_for_its_sources_and_plan(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: "abc")
    _summary(tmp_path, "abc", "config 7 split 2,1")
    assert bench.measured_traffic("k", "wl", 8, "config 7 split 2,1") == 123456789
    assert bench.measured_traffic("k", "wl", 8, "config 3 split 2,1") is None     # other plan
    assert bench.measured_traffic("k", "wl", 9, "config 7 split 2,1") is None     # no summary
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: "def")
    assert bench.measured_traffic("k", "wl", 8, "config 7 split 2,1") is None     # other sources


def test_stream_ordered_search_includes_the_rules_configurations():
    """The fastest-pair search covers the configurations the rules would
    plan (a tuned plan's configuration is added to the search at run time)."""
    from consumer_gemm_chain_amd import mlp_chain as mc
    for wl in (1, 2, 3, 4):
        w = gen.WORKLOADS[wl]
        for M in w.Ms:
            p = mc.mlp_chain_plan(M, w.H, w.I, mc.ACTS[w.act], mc.MLP_POLICY_STREAM_ORDERED, -256)
            assert p["config"] in bench.so_search_configs(M), (w.name, M, p)
    assert (1, 1) in bench.SO_SPLITS and (2, 1) in bench.SO_SPLITS


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_sweep_summary_of_every_workload_stays_small():
    """The stdout line carries one compact row per (workload, M) of the
    tile_sync sweep; with every workload's M list it stays well under the
    few KB the driver reads back."""
    import json
    rows = []
    for wl in (1, 2, 3, 4):
        w = gen.WORKLOADS[wl]
        for M in w.Ms:
            for pol in ("stream_ordered", "row_sync", "tile_sync"):
                rows.append({"workload": w.name, "M": M, "policy": pol, "us": 1234.5678, "us_cold": 1234.5678,
                             "stream_ordered_best": {"us": 1234.5678, "us_cold": 1234.5678},
                             "speedup_vs_stream_ordered_best": 1.02345, "speedup_vs_stream_ordered_best_cold": 1.02345,
                             "speedup_vs_stream_ordered": 1.02345, "roofline_frac_cold": 0.43219,
                             "roofline_frac_cold_written": 0.43219, "bound": "mfma"})
    s = bench.sweep_summary(rows)
    assert len(s) == sum(len(gen.WORKLOADS[wl].Ms) for wl in (1, 2, 3, 4))
    assert all(len(r) == len(bench.SUMMARY_COLUMNS) for r in s)
    assert len(json.dumps(s, separators=(",", ":"))) < 2000


def test_sweep_reps_follow_the_timing_protocol():
    assert bench.sweep_reps(1, 0) >= 50 and bench.sweep_reps(512, 0) >= 50
    assert bench.sweep_reps(2048, 0) >= 10
    assert bench.sweep_reps(2048, 7) == 7
