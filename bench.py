"""Benchmark of the tile-synchronized MLP GEMM chain on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--M 2048]
                    [--policy tile_sync] [--no-sweep] [--no-cpu] [--sweep-reps R]

A step is one chain pass (GEMM1 + activation, then GEMM2) over one batch of
M tokens, enqueued through the C ABI (mlp_chain_run) with inputs already
resident in HBM.  The headline is the GPT-3 175B MLP shard (H=12288,
I=6144, fp16, GeLU; the pages' GPT-3 MLP under 8-way model parallelism) at
M=2048 tokens with the tile_sync policy.  Next to it the script reports two
stream-ordered two-kernel baselines: the planned pair, which shares the fused
run's K split and is its bit-exact reference, and the fastest pair over tile
configurations and K splits (the fair speed baseline), also replayed as a
HIP graph (the pair without host launch gaps).  It also reports a
sweep of the three policies over each workload's M list (GPT-3 up to --M,
the LLaMA-65, Llama-2 and 8192^3 shapes in full): time hot and with the
Infinity Cache flushed, TFLOP/s, fraction of the MFMA / HBM roofline,
speedup over both stream-ordered baselines, and an overhead in the style of
the FLUX summary card's Effective Communication Time (policy time minus the
best isolated GEMM1 and GEMM2 times).  Then the dominant kernel's roofline
position measured with HIP events, and the CPU oracle timed on a bounded
sample of rows.

Prints ONE short JSON line on stdout (a few KB: the headline, the
baselines, the roofline position, the CPU baseline and a compact table of
the sweep); the full per-policy sweep rows go to stderr, one JSON object per
line, and to --sweep-out if given.  Inputs are seeded synthetic data of the
workload's shapes (no trained weights).

    python bench.py --kernels-only     only the headline policy and the planned
                                       stream-ordered pair (for profiler runs)
    python bench.py --copy-mib 1024    only a device copy of that size, three
                                       times (calibration of the memory-traffic
                                       counters: FETCH_SIZE / WRITE_SIZE of a
                                       copy of known size)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # MI355X dense fp16 / bf16 matrix peak
PEAK_HBM_GBS = 8000.0                                  # MI355X HBM3E bandwidth
POLICIES = ("stream_ordered", "row_sync", "tile_sync")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def roofline_time_us(w, M, dtype):
    f = w.flops(M)
    b = w.bytes(M)
    t_mfma = f / (PEAK_MFMA_TFLOPS[dtype] * 1e12) * 1e6
    t_hbm = b / (PEAK_HBM_GBS * 1e9) * 1e6
    return max(t_mfma, t_hbm), ("mfma" if t_mfma >= t_hbm else "hbm")


KERNEL_SOURCES = ("chain_configs.h", "chain_device.hpp", "chain_kernels.hip")


def kernel_sources_hash() -> str:
    """Short hash of the device sources: a counter summary taken on other
    sources no longer describes the kernels and is not used."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "consumer_gemm_chain_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, M: int, plan: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_<workload>_M<M>_traffic.md (FETCH_SIZE + WRITE_SIZE
    scaled by the copy calibration), or None when there is no summary or it
    was taken on other kernel sources or another plan (tile configuration and
    K split, e.g. "config 8 split 2,1")."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_M{M}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":", 1)[0].strip() in ("sources", "plan", "traffic_bytes_per_launch"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if (fields.get("sources") != kernel_sources_hash() or fields.get("plan") != plan
            or "traffic_bytes_per_launch" not in fields):
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def weight_strides(w, dense: bool):
    """Row strides (elements) of the workload's device weights: the
    library's preferred padded strides (rows an odd number of 128-byte
    lines apart), or dense rows."""
    from consumer_gemm_chain_amd import mlp_chain as mc
    g = 2 if w.act == "swiglu" else 1
    return (g * w.I, w.H) if dense else mc.mlp_chain_weight_ld(w.H, w.I, mc.ACTS[w.act])


class Runner:
    """Device inputs for one workload at its largest M; runs slice X rows.
    The weights live in rows `ld` apart (weight_strides), and every chain
    made here is told so."""

    def __init__(self, w, max_M, dense_weights=False):
        import torch
        from consumer_gemm_chain_amd import gen
        from consumer_gemm_chain_amd.tensors import to_dev, to_dev_rows
        self.w = w
        t0 = time.time()
        w1, w2 = gen.weights(w)
        x = gen.x_rows(w, max_M, max_M=max(max_M, w.max_M))
        self.host = (x, w1, w2)
        self.ld = weight_strides(w, dense_weights)
        self.x = to_dev(x, w.dtype)
        self.w1 = to_dev_rows(w1, w.dtype, self.ld[0])
        self.w2 = to_dev_rows(w2, w.dtype, self.ld[1])
        dt = self.x.dtype
        self.out = torch.empty((max_M, w.H), dtype=dt, device="cuda")
        torch.cuda.synchronize()
        log(f"inputs for {w.name} (M<={max_M}) ready in {time.time() - t0:.1f}s")

    def chain(self, M, policy, layers=1):
        from consumer_gemm_chain_amd.mlp_chain import MlpChain
        ch = MlpChain(M, self.w.H, self.w.I, self.w.act, self.w.dtype, policy, layers=layers)
        ch.set_weight_ld(*self.ld)
        return ch

    def args(self, M):
        return self.x[:M], self.w1, self.w2, self.out[:M]


def event_times(fn, n, stream, flush=None):
    """Per-call device times (us) from HIP events recorded on `stream`."""
    import torch
    ts = []
    for _ in range(n):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return np.array(ts)


def sweep_reps(M, reps):
    """Timed runs per point: at least 50 where a run is short (M <= 512),
    20 otherwise, unless --sweep-reps fixes the count."""
    if reps > 0:
        return reps
    return 50 if M <= 512 else 20


def cache_flushes(flush_buf):
    """The two ways of emptying the 256 MB Infinity Cache between timed runs.

    "clean" reads the 512 MB buffer: the cache ends up holding clean lines of
    it and none of the weights.  "written" adds one to every byte of it: the
    cache ends up holding 256 MB of dirty lines, whose write-back to HBM then
    overlaps the timed run's first reads (a plain read of LLaMA-65's W1
    panels ran at 2.7 TB/s after it against 4.3-4.7 TB/s after the clean
    flush), so that figure also charges the run for the flush's own writes."""
    import torch
    flat = flush_buf.view(torch.float32)
    return {"clean": lambda: flat.sum(), "written": lambda: flush_buf.add_(1)}


def sweep(runner, Ms, reps, stream, flush_buf):
    """Per (M, policy): median event time hot (weights left in the caches by
    the previous run), cold (a 512 MB buffer read between runs, so the 256 MB
    Infinity Cache holds none of the weights) and cold after a written flush
    (the same buffer rewritten, which leaves dirty lines to be written back
    during the run), TFLOP/s, roofline fraction, speedup over both
    stream-ordered baselines, and the ECT-style overhead against the best
    isolated GEMM1 + GEMM2 times (hot)."""
    import torch
    w = runner.w
    flushes = cache_flushes(flush_buf)
    flush, flush_w = flushes["clean"], flushes["written"]
    rows = []
    for M in Ms:
        n = sweep_reps(M, reps)
        x, w1, w2, out = runner.args(M)
        res = {}
        with runner.chain(M, "stream_ordered") as so:
            for _ in range(3):
                so.run_phase(1, x=x, w1=w1)
                so.run_phase(2, w2=w2, out=out)
            torch.cuda.synchronize()
            g1 = np.median(event_times(lambda: so.run_phase(1, x=x, w1=w1), n, stream))
            g2 = np.median(event_times(lambda: so.run_phase(2, w2=w2, out=out), n, stream))
        for pol in POLICIES:
            with runner.chain(M, pol) as ch:
                for _ in range(3):
                    ch.run(x, w1, w2, out)
                torch.cuda.synchronize()
                ts = event_times(lambda: ch.run(x, w1, w2, out), n, stream)
                tc = event_times(lambda: ch.run(x, w1, w2, out), n, stream, flush)
                tw = event_times(lambda: ch.run(x, w1, w2, out), n, stream, flush_w)
                assert ch.status() == 0
                info = ch.info()
            res[pol] = (float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90)),
                        float(np.median(tc)), info, float(np.median(tw)))
        t_roof, bound = roofline_time_us(w, M, w.dtype)
        t_so, t_so_cold = res["stream_ordered"][0], res["stream_ordered"][3]
        t_best, b_cfg, b_s1, b_s2 = best_stream_ordered(runner, M, stream, max(5, n // 4))
        with runner.chain(M, "stream_ordered") as sb:
            sb.set_config(b_cfg)
            sb.set_split(b_s1, b_s2)
            sb.run(x, w1, w2, out)
            t_best = min(t_best, float(np.median(event_times(lambda: sb.run(x, w1, w2, out), n, stream))))
            t_best_cold = float(np.median(event_times(lambda: sb.run(x, w1, w2, out), n, stream, flush)))
            t_best_written = float(np.median(event_times(lambda: sb.run(x, w1, w2, out), n, stream, flush_w)))
        # the planned pair is one of the searched plans: the fastest is never slower than it
        so_info = res["stream_ordered"][4]
        if t_so < t_best:
            t_best, b_cfg, b_s1, b_s2 = t_so, so_info["config"], so_info["S1"], so_info["S2"]
        t_best_cold = min(t_best_cold, t_so_cold)
        t_best_written = min(t_best_written, res["stream_ordered"][5])
        for pol in POLICIES:
            t, p10, p90, tcold, info, twritten = res[pol]
            rows.append({
                "workload": w.name, "M": M, "policy": pol, "reps": n,
                "us": round(t, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2),
                "us_cold": round(tcold, 2), "us_cold_written": round(twritten, 2),
                "tflops": round(w.flops(M) / (t * 1e-6) / 1e12, 2),
                "tflops_cold": round(w.flops(M) / (tcold * 1e-6) / 1e12, 2),
                "gbs": round(w.bytes(M) / (t * 1e-6) / 1e9, 1),
                "gbs_cold": round(w.bytes(M) / (tcold * 1e-6) / 1e9, 1),
                "roofline_frac": round(t_roof / t, 4), "roofline_frac_cold": round(t_roof / tcold, 4),
                "roofline_frac_cold_written": round(t_roof / twritten, 4),
                "bound": bound,
                "speedup_vs_stream_ordered": round(t_so / t, 4),
                "speedup_vs_stream_ordered_best": round(t_best / t, 4),
                "speedup_vs_stream_ordered_cold": round(t_so_cold / tcold, 4),
                "speedup_vs_stream_ordered_best_cold": round(t_best_cold / tcold, 4),
                "speedup_vs_stream_ordered_best_cold_written": round(t_best_written / twritten, 4),
                "stream_ordered_best": {"us": round(t_best, 2), "us_cold": round(t_best_cold, 2),
                                        "us_cold_written": round(t_best_written, 2),
                                        "config": b_cfg, "S1": b_s1, "S2": b_s2},
                "overhead_vs_best_unsplit_us": round(t - (g1 + g2), 2),
                "tiles": [info["T1"], info["T2"]], "tile": [info["BM"], info["BN1"]],
                "config": info["config"], "split": [info["S1"], info["S2"]],
            })
            log(json.dumps(rows[-1]))
        log(f"{w.name} M={M:5d} g1={g1:8.1f}us g2={g2:8.1f}us  " + "  ".join(
            f"{p}={res[p][0]:8.1f}/{res[p][3]:8.1f}/{res[p][5]:8.1f}us" for p in POLICIES)
            + f"  best stream_ordered={t_best:8.1f}/{t_best_cold:8.1f}/{t_best_written:8.1f}us"
            + f" (config {b_cfg}, split {b_s1},{b_s2})  (hot/cold/cold after a written flush)")
    return rows


# Columns of the compact sweep table in the stdout line (one row per
# workload and M, for the tile_sync policy).
SUMMARY_COLUMNS = ("workload", "M", "tile_sync_us", "tile_sync_us_cold", "best_pair_us", "best_pair_us_cold",
                   "speedup_vs_best_pair", "speedup_vs_best_pair_cold", "speedup_vs_same_split_pair",
                   "roofline_frac_cold", "roofline_frac_cold_written", "bound")
SHORT_NAMES = {"tiny_gelu_f16": "tiny", "gpt3_175b_mlp_tp8_f16": "gpt3", "llama65b_swiglu_tp8_f16": "llama65",
               "llama2_70b_swiglu_tp8_bf16": "llama2", "stress_square_chain_bf16": "stress8192"}


def sweep_summary(rows):
    out = []
    for r in rows:
        if r["policy"] != "tile_sync":
            continue
        b = r["stream_ordered_best"]
        out.append([SHORT_NAMES.get(r["workload"], r["workload"]), r["M"], round(r["us"], 1),
                    round(r["us_cold"], 1), round(b["us"], 1), round(b["us_cold"], 1),
                    round(r["speedup_vs_stream_ordered_best"], 3), round(r["speedup_vs_stream_ordered_best_cold"], 3),
                    round(r["speedup_vs_stream_ordered"], 3), round(r["roofline_frac_cold"], 3),
                    round(r["roofline_frac_cold_written"], 3), r["bound"]])
    return out


SO_SPLITS = tuple((s1, s2) for s1 in (1, 2, 3, 4) for s2 in (1, 2))


def so_search_configs(M):
    """Tile configurations the best stream-ordered plan is searched over."""
    return (0, 4, 9) if M <= 16 else (3, 4, 8, 10) if M <= 256 else (3, 7, 8, 10) if M <= 512 else (3, 7, 8)


def best_stream_ordered(runner, M, stream, reps):
    """The fastest stream-ordered pair over tile configurations x K splits
    (S1 in 1..4, S2 in 1..2, plus the planned split): (median event us,
    config, S1, S2).  Every one of these plans is a valid stream-ordered
    baseline; only the plan whose split the fused policies share is
    bit-identical to them."""
    import torch
    x, w1, w2, out = runner.args(M)
    with runner.chain(M, "stream_ordered") as so:
        planned = (so.info()["S1"], so.info()["S2"])
        planned_cfg = so.info()["config"]
    best = None
    for cfg in sorted(set(so_search_configs(M)) | {planned_cfg}):
        for s1, s2 in sorted(set(SO_SPLITS) | {planned}):
            with runner.chain(M, "stream_ordered") as so:
                so.set_config(cfg)
                so.set_split(s1, s2)
                for _ in range(2):
                    so.run(x, w1, w2, out)
                torch.cuda.synchronize()
                t = float(np.median(event_times(lambda: so.run(x, w1, w2, out), reps, stream)))
                assert so.status() == 0
            if best is None or t < best[0]:
                best = (t, cfg, s1, s2)
    return best


LAYER_MS = (16, 256, 2048)


def layers_sweep(w, L, Ms, reps, stream, ld):
    """A chain of L MLP layers of the workload's shapes (own seeded weights
    per layer) at each M: the fused policies' single persistent kernel
    against the 2L stream-ordered kernels, event medians (hot).  The fused
    kernel overlaps each layer's consumers with the previous layer's tail."""
    import torch
    from consumer_gemm_chain_amd import gen
    from consumer_gemm_chain_amd.mlp_chain import MlpChain
    from consumer_gemm_chain_amd.tensors import to_dev, to_dev_rows
    g = 2 if w.act == "swiglu" else 1
    w1s = [to_dev_rows(gen.normal_bits((w.H, g * w.I), 9000 + 10 * l, w.w_scale, w.dtype), w.dtype, ld[0])
           for l in range(L)]
    w2s = [to_dev_rows(gen.normal_bits((w.I, w.H), 9001 + 10 * l, w.w_scale, w.dtype), w.dtype, ld[1])
           for l in range(L)]
    xs = to_dev(gen.x_rows(w, max(Ms)), w.dtype)
    out = torch.empty((max(Ms), w.H), dtype=xs.dtype, device="cuda")
    rows = []
    for M in Ms:
        t = {}
        for pol in POLICIES:
            with MlpChain(M, w.H, w.I, w.act, w.dtype, pol, layers=L) as ch:
                ch.set_weight_ld(*ld)
                for _ in range(3):
                    ch.run_layers(xs[:M], w1s, w2s, out[:M])
                torch.cuda.synchronize()
                t[pol] = float(np.median(event_times(lambda: ch.run_layers(xs[:M], w1s, w2s, out[:M]),
                                                     sweep_reps(M, reps), stream)))
                assert ch.status() == 0
        rows.append([M, round(t["tile_sync"], 1), round(t["row_sync"], 1), round(t["stream_ordered"], 1),
                     round(t["stream_ordered"] / t["tile_sync"], 3),
                     round(L * w.flops(M) / (t["tile_sync"] * 1e-6) / 1e12, 1)])
        log(f"{L} layers of {w.name} M={M}: tile_sync {t['tile_sync']:.1f} us, row_sync {t['row_sync']:.1f} us, "
            f"{2 * L} stream-ordered kernels {t['stream_ordered']:.1f} us")
    return rows


def host_cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(runner, M, budget_s=12.0):
    """The oracle as it stands, on a bounded sample of the workload's rows."""
    from oracle import oracle
    w = runner.w
    x, w1, w2 = runner.host
    threads = oracle.max_threads()
    R = max(1, min(M, threads))
    while True:
        t0 = time.perf_counter()
        oracle.mlp_chain(x[:R], w1, w2, w.act, w.dtype)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 3 or R >= M:
            break
        R = min(M, R * 2)
    tflops = w.flops(R) / dt / 1e12
    return {"value": round(tflops, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": host_cpu_model(),
            "sample": f"{w.name}: first {R} of {M} rows in one call ({dt:.2f} s, weights widened "
                      f"inside the call), throughput scaled per row"}


def copy_calibration(mib: int, reps: int = 3) -> None:
    """A plain device-to-device copy of `mib` MiB, `reps` times: under
    rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) each copy dispatch reads and
    writes exactly that many bytes, which calibrates the counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB x {reps}")


def timed_loop(ch, args, steps, stream):
    """Host wall time of `steps` back-to-back runs, and each run's event time."""
    import torch
    x, w1, w2, out = args
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        ch.run(x, w1, w2, out)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return wall, kern


def roofline_entry(w, M, policy, info, kern_us):
    """Roofline position of the dominant kernel from its mean event time."""
    F = w.flops(M)
    t_roof, bound = roofline_time_us(w, M, w.dtype)
    achieved = F / (kern_us * 1e-6) / 1e12
    roof = {"bound": bound,
            "kernel": f"chain_persistent_kernel ({policy})" if policy != "stream_ordered"
            else "gemm1_act_kernel + gemm2_kernel",
            "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS[w.dtype], "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MFMA_TFLOPS[w.dtype], 4),
            "kernel_us": round(kern_us, 2),
            "traffic": measured_traffic("chain_persistent_kernel" if policy != "stream_ordered" else "gemm_pair",
                                        w.name, M, f"config {info['config']} split {info['S1']},{info['S2']}"),
            "algorithmic_flops_per_launch": F, "algorithmic_bytes_per_launch": w.bytes(M),
            "roofline_time_us": round(t_roof, 2), "frac_of_roofline_time": round(t_roof / kern_us, 4)}
    if bound == "hbm":
        gbs = w.bytes(M) / (kern_us * 1e-6) / 1e9
        roof.update({"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4)})
    return roof


def graph_replay_time(runner, M, plan, steps, warmup, stream, policy="stream_ordered"):
    """Wall time of `steps` replays of one run of `policy` (the stream-ordered
    pair, or a fused run), with the plan (config, S1, S2) or the planned one
    (plan None), captured as a HIP graph: the same kernels without host
    launch gaps (no launch depends on anything the host changes per run)."""
    import torch
    x, w1, w2, out = runner.args(M)
    with runner.chain(M, policy) as sg:
        if plan is not None:
            sg.set_config(plan[0])
            sg.set_split(plan[1], plan[2])
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(3):
                sg.run(x, w1, w2, out)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sg.run(x, w1, w2, out)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        assert sg.status() == 0
        del graph
    return wall


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--M", type=int, default=2048)
    ap.add_argument("--policy", default="tile_sync", choices=POLICIES)
    ap.add_argument("--sweep-reps", type=int, default=0,
                    help="timed runs per sweep point (0: 50 for M <= 512, else 20)")
    ap.add_argument("--sweep-workloads", default="1,2,3,4",
                    help="workloads swept over their M lists (the headline workload up to --M)")
    ap.add_argument("--sweep-out", default=None, help="also write the full sweep rows to this JSON file")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--layers", type=int, default=2,
                    help="MLP layers of the multi-layer chain timed after the sweep (0: none)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work the CPU baseline aims at (bounded sample of rows)")
    ap.add_argument("--kernels-only", action="store_true",
                    help="only the headline policy and the planned stream-ordered pair (profiler runs)")
    ap.add_argument("--dense-weights", action="store_true",
                    help="weights in dense rows instead of the library's preferred padded row strides")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only a device copy of this many MiB, three times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the chain runs on one MI355X; no sharding); "
              f"got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    from consumer_gemm_chain_amd import gen
    from consumer_gemm_chain_amd.mlp_chain import load_library
    load_library()   # fails loudly if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_mib > 0:
        copy_calibration(args.copy_mib)
        return

    w = gen.WORKLOADS[args.workload]
    M = args.M
    quick = args.kernels_only
    sweep_Ms = [m for m in w.Ms if m <= M] if not (args.no_sweep or quick) else []
    runner = Runner(w, max(M, max(sweep_Ms) if sweep_Ms else M), args.dense_weights)
    stream = torch.cuda.current_stream()
    hargs = runner.args(M)
    x, w1, w2, out = hargs

    # The stream-ordered two-kernel baselines are timed both before and
    # after the headline block, and the faster of the two blocks counts: the
    # GPU clock drifts with power and temperature over a run (1.7 - 2.1 GHz
    # measured), which would otherwise favour whichever policy runs first,
    # and a block disturbed by anything else on the machine must not make
    # the baseline look slow.  The fastest
    # stream-ordered plan (any tile configuration and K split) is the fair
    # baseline; the planned one shares the fused policies' split and is
    # their bit-exact reference.
    so = runner.chain(M, "stream_ordered")
    so_best = None
    if not quick:
        _, bcfg, bs1, bs2 = best_stream_ordered(runner, M, stream, 10)
        so_best = runner.chain(M, "stream_ordered")
        so_best.set_config(bcfg)
        so_best.set_split(bs1, bs2)
    for _ in range(args.warmup):
        so.run(*hargs)
        if so_best:
            so_best.run(*hargs)
    wall_so_a, kern_so_a = timed_loop(so, hargs, args.steps, stream)
    if so_best:
        wall_sb_a, kern_sb_a = timed_loop(so_best, hargs, args.steps, stream)

    # headline: the chosen policy, K timed steps after W warmup steps
    with runner.chain(M, args.policy) as ch:
        for _ in range(args.warmup):
            ch.run(*hargs)
        wall, kern = timed_loop(ch, hargs, args.steps, stream)
        assert ch.status() == 0, "device watchdog fired during the timed steps"
        info = ch.info()
    ms_per_step = wall / args.steps * 1e3
    F = w.flops(M)
    value = F / (ms_per_step * 1e-3) / 1e12

    wall_so_b, kern_so_b = timed_loop(so, hargs, args.steps, stream)
    so_info = so.info()
    so.close()
    wall_so, kern_so = min((wall_so_a, kern_so_a), (wall_so_b, kern_so_b), key=lambda p: p[0])
    so_tflops = F / (wall_so / args.steps) / 1e12
    if so_best:
        wall_sb_b, kern_sb_b = timed_loop(so_best, hargs, args.steps, stream)
        so_best.close()
        wall_sb, kern_sb = min((wall_sb_a, kern_sb_a), (wall_sb_b, kern_sb_b), key=lambda p: p[0])
        if wall_so < wall_sb:
            # the planned pair is one of the searched plans: the fastest is never slower than it
            wall_sb, kern_sb = wall_so, kern_so
            bcfg, bs1, bs2 = so_info["config"], so_info["S1"], so_info["S2"]
        sb_tflops = F / (wall_sb / args.steps) / 1e12

    roofline = roofline_entry(w, M, args.policy, info, float(np.mean(kern)))
    roofline["kernel_us_p10_p90"] = [round(float(np.percentile(kern, 10)), 2),
                                     round(float(np.percentile(kern, 90)), 2)]

    line = {
        "metric": "MLP-chain TFLOP/s and % roofline vs stream-ordered 2-kernel, M=1..2048",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "M": M, "H": w.H, "I": w.I, "act": w.act, "policy": args.policy,
                   "tile": [info["BM"], info["BN1"], info["BK"]], "tiles": [info["T1"], info["T2"]],
                   "tile_config": info["config"], "split": [info["S1"], info["S2"]],
                   "grid": info["grid"], "weight_ld": list(runner.ld), "parallelism": "single GPU"},
        "stream_ordered": {"value": round(so_tflops, 2), "ms_per_step": round(wall_so / args.steps * 1e3, 4),
                           "kernel_pair_us": round(float(np.mean(kern_so)), 2),
                           "plan": [so_info["config"], so_info["S1"], so_info["S2"]],
                           "note": "planned pair [config, S1, S2]: the fused run's K split (bit-exact reference)"},
        "speedup_vs_stream_ordered": round(value / so_tflops, 4),
        "roofline": roofline,
    }

    if not quick:
        line["stream_ordered_best"] = {
            "value": round(sb_tflops, 2), "ms_per_step": round(wall_sb / args.steps * 1e3, 4),
            "kernel_pair_us": round(float(np.mean(kern_sb)), 2), "plan": [bcfg, bs1, bs2],
            "note": f"fastest pair over configs {list(so_search_configs(M))} x splits S1 1..4, S2 1..2"}
        line["speedup_vs_stream_ordered_best"] = round(value / sb_tflops, 4)
        wall_sgraph = graph_replay_time(runner, M, (bcfg, bs1, bs2), args.steps, args.warmup, stream)
        sgraph_tflops = F / (wall_sgraph / args.steps) / 1e12
        line["stream_ordered_graph"] = {"value": round(sgraph_tflops, 2),
                                        "ms_per_step": round(wall_sgraph / args.steps * 1e3, 4),
                                        "plan": [bcfg, bs1, bs2],
                                        "note": "fastest pair captured as a HIP graph and replayed"}
        line["speedup_vs_stream_ordered_graph"] = round(value / sgraph_tflops, 4)
        wall_pgraph = graph_replay_time(runner, M, None, args.steps, args.warmup, stream, args.policy)
        line["policy_graph"] = {"value": round(F / (wall_pgraph / args.steps) / 1e12, 2),
                                "ms_per_step": round(wall_pgraph / args.steps * 1e3, 4),
                                "note": f"{args.policy} captured as a HIP graph and replayed"}

    rows = []
    flush_buf = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda") if sweep_Ms else None
    if sweep_Ms:
        rows += sweep(runner, sweep_Ms, args.sweep_reps, stream, flush_buf)

    line["cpu_baseline"] = None if (args.no_cpu or quick) else cpu_baseline(runner, M, args.cpu_budget)

    if sweep_Ms:
        for wl in (int(v) for v in args.sweep_workloads.split(",") if v.strip()):
            if wl == args.workload:
                continue
            del runner
            torch.cuda.empty_cache()
            ws = gen.WORKLOADS[wl]
            runner = Runner(ws, ws.max_M, args.dense_weights)
            rows += sweep(runner, list(ws.Ms), args.sweep_reps, stream, flush_buf)
    del flush_buf

    layer_Ms = [m for m in LAYER_MS if m <= M]
    if sweep_Ms and args.layers > 1 and layer_Ms:
        del runner
        torch.cuda.empty_cache()
        line["layers"] = {"workload": w.name, "layers": args.layers,
                          "columns": ["M", "tile_sync_us", "row_sync_us", "stream_ordered_us",
                                      "speedup_vs_stream_ordered", "tile_sync_tflops"],
                          "rows": layers_sweep(w, args.layers, layer_Ms, args.sweep_reps, stream,
                                               weight_strides(w, args.dense_weights))}

    if rows:
        line["sweep_columns"] = list(SUMMARY_COLUMNS)
        line["sweep"] = sweep_summary(rows)
        line["sweep_note"] = ("tile_sync event medians hot / cold (512 MB read between runs; _written: 512 MB "
                              "written); best pair: fastest stream-ordered plan; all rows on stderr")
    if args.sweep_out:
        with open(args.sweep_out, "w") as fh:
            json.dump(rows, fh, indent=1)
    print(json.dumps(line, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
