"""rocprofv3 harness of the MLP GEMM chain: kernel durations, matrix-core
utilisation and memory traffic of the benchmark's kernels, written as short
text summaries.

    python rocprof_harness.py [--workload 1] [--M 2048] [--policy tile_sync]
                              [--raw-dir gpurun_out/prof] [--summary-dir profiles]

Each measurement is its own profiler run of `bench.py --kernels-only` (the
headline policy's persistent kernel and the planned stream-ordered pair,
nothing else), every run under a hard time limit:
  * kernel trace + stats           -> <summary-dir>/chain_kernels_<wl>_M<M>_trace.txt
  * SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES, GRBM_GUI_ACTIVE
                                   -> <summary-dir>/chain_kernels_<wl>_M<M>_mfma.md
  * FETCH_SIZE, then WRITE_SIZE (one counter group per run), and the same
    two counters over a 1 GiB device copy (`bench.py --copy-mib 1024`),
    whose known size calibrates them
                                   -> <summary-dir>/chain_persistent_kernel_<wl>_M<M>_traffic.md
The traffic summary records the kernel sources' hash and the plan, so that
bench.py reports it as the roofline's `traffic` only while both still hold.
Matrix-core utilisation and HBM bytes per second follow from the counters and
the profiled durations; at small M (weight streaming) the GB/s figure is the
one that matters, at large M the matrix-core one.

The harness itself never touches the GPU: it only starts the profiler runs
as child processes and parses their CSV output.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_MIB = 1024
SIMDS = 1024          # MI355X: 256 CUs x 4 SIMDs
CUS = 256
XCDS = 8


def _run(cmd, log_path, limit_s):
    """One profiler run under a hard time limit; returns its exit status."""
    full = ["timeout", "-s", "KILL", str(limit_s)] + cmd
    print("+ " + " ".join(full), flush=True)
    with open(log_path, "w") as log:
        r = subprocess.run(full, stdout=log, stderr=subprocess.STDOUT, cwd=ROOT)
    print(f"  exit {r.returncode} ({log_path})", flush=True)
    return r.returncode


def _find(raw, name, suffix):
    hits = glob.glob(os.path.join(raw, name, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {os.path.join(raw, name)}")
    return hits[0]


def _counters(path):
    """{dispatch id: (kernel, workgroups, duration us, {counter: value})}"""
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        if d not in out:
            wg = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            out[d] = (r["Kernel_Name"], wg, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3, {})
        c = out[d][3]
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def short_name(k):
    """`chain_persistent_kernel<256, 256, 2, 4, 2, 2>` from the demangled name."""
    base = k.split("(")[0].split("<")[0].split("::")[-1]
    if "TileCfg<" in k:
        return base + "<" + k.split("TileCfg<")[1].split(">")[0] + ">"
    return base


def _chain_rows(disp):
    """Dispatches of the chain's kernels grouped by (kernel, workgroups)."""
    g = collections.defaultdict(list)
    for kname, wg, dur, c in disp.values():
        if "mlpc::" in kname:
            g[(short_name(kname), wg)].append((dur, c))
    return g


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--M", type=int, default=2048)
    ap.add_argument("--policy", default="tile_sync")
    ap.add_argument("--raw-dir", default=os.path.join("gpurun_out", "prof"))
    ap.add_argument("--summary-dir", default="profiles")
    args = ap.parse_args()

    from consumer_gemm_chain_amd import gen
    import bench
    w = gen.WORKLOADS[args.workload]
    tag = f"{w.name}_M{args.M}"
    raw = os.path.join(args.raw_dir, tag)
    os.makedirs(raw, exist_ok=True)
    os.makedirs(args.summary_dir, exist_ok=True)
    py = sys.executable or "python3"
    bench_cmd = [py, "bench.py", "--kernels-only", "--workload", str(args.workload), "--M", str(args.M),
                 "--policy", args.policy]
    prof = ["rocprofv3", "--output-format", "csv"]

    def run(name, extra, program, limit):
        cmd = prof + ["-d", os.path.join(raw, name), "-o", name] + extra + ["--"] + program
        rc = _run(cmd, os.path.join(raw, name + ".log"), limit)
        if rc != 0:
            raise SystemExit(f"profiler run {name} ended with status {rc}; see {raw}/{name}.log")

    # 1. kernel trace + stats; the bench line of the same run goes to kt.log
    run("kt", ["--kernel-trace", "--stats"], bench_cmd + ["--steps", "10", "--warmup", "3"], 300)
    # 2. matrix-core activity and clock
    run("mfma", ["--pmc", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"],
        bench_cmd + ["--steps", "3", "--warmup", "1"], 300)
    # 3. memory traffic, one counter per run, and the copy calibration
    run("fetch", ["--pmc", "FETCH_SIZE"], bench_cmd + ["--steps", "3", "--warmup", "1"], 300)
    run("write", ["--pmc", "WRITE_SIZE"], bench_cmd + ["--steps", "3", "--warmup", "1"], 300)
    copy_cmd = [py, "bench.py", "--copy-mib", str(COPY_MIB)]
    run("cfetch", ["--pmc", "FETCH_SIZE"], copy_cmd, 120)
    run("cwrite", ["--pmc", "WRITE_SIZE"], copy_cmd, 120)

    cmds = "\n".join(f"    {c}" for c in (
        "python rocprof_harness.py " + " ".join(sys.argv[1:]),
        f"  -> rocprofv3 --kernel-trace --stats -- {' '.join(bench_cmd[1:])} --steps 10 --warmup 3",
        f"  -> rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE -- "
        f"{' '.join(bench_cmd[1:])} --steps 3 --warmup 1",
        f"  -> rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- {' '.join(bench_cmd[1:])} --steps 3 --warmup 1",
        f"  -> rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- bench.py --copy-mib {COPY_MIB}"))
    sources = bench.kernel_sources_hash()
    bench_line = None
    for line in open(os.path.join(raw, "kt.log")):
        if line.startswith("{") and '"metric"' in line:
            bench_line = json.loads(line)
    if bench_line is None:
        raise SystemExit("the traced bench run printed no JSON line")
    cfgd = bench_line["config"]
    plan = f"config {cfgd['tile_config']} split {cfgd['split'][0]},{cfgd['split'][1]}"
    so_plan = bench_line["stream_ordered"]["plan"]
    header = (f"workload: {w.name} (H={w.H}, I={w.I}, {w.act}, {w.dtype}), M={args.M}\n"
              f"policy: {args.policy}, tile {cfgd['tile']}, {plan}; planned stream-ordered pair: "
              f"config {so_plan[0]} split {so_plan[1]},{so_plan[2]}\n"
              f"weights: rows {cfgd.get('weight_ld', ['dense', 'dense'])[0]} (W1) and "
              f"{cfgd.get('weight_ld', ['dense', 'dense'])[1]} (W2) elements apart\n"
              f"sources: {sources}\n")

    # ---- trace
    rows = list(csv.DictReader(open(_find(raw, "kt", "kernel_stats.csv"))))
    lines = [f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
             f"{float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):8.2f}  {short_name(r['Name'])}" for r in rows]
    pers = [r for r in rows if "persistent" in r["Name"]]
    prof_avg = float(pers[0]["AverageNs"]) / 1e3 if pers else None
    trace = (f"# Kernel durations, {tag}\n\ncommands (repository root, one MI355X):\n{cmds}\n\n{header}\n"
             f" calls     avg_us     min_us     max_us  total_%  kernel\n" + "\n".join(lines) + "\n\n"
             f"Bench line of the traced run (HIP events on the launch stream, timed steps only):\n"
             f"    {args.policy} kernel_us = {bench_line['roofline']['kernel_us']}"
             + (f"   (profiler average of all its launches, warmup included: {prof_avg:.1f})" if prof_avg else "")
             + f"\n    value = {bench_line['value']} TFLOP/s; planned stream-ordered pair kernel_us = "
             f"{bench_line['stream_ordered']['kernel_pair_us']}\n")
    with open(os.path.join(args.summary_dir, f"chain_kernels_{tag}_trace.txt"), "w") as fh:
        fh.write(trace)

    # ---- matrix cores and clock
    mf = _chain_rows(_counters(_find(raw, "mfma", "counter_collection.csv")))
    mrows = []
    for (k, wg), ds in sorted(mf.items()):
        dur = statistics.median(d for d, _ in ds)
        cyc = statistics.median(c["GRBM_GUI_ACTIVE"] / XCDS for _, c in ds)
        busy = statistics.median(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * c["GRBM_GUI_ACTIVE"] / XCDS) for _, c in ds)
        cu = statistics.median(c["SQ_BUSY_CU_CYCLES"] / (CUS * c["GRBM_GUI_ACTIVE"] / XCDS) for _, c in ds)
        mrows.append(f"| {k} | {wg} | {len(ds)} | {dur:.1f} | {cyc / dur / 1e3:.2f} | {busy:.3f} | {cu:.2f} |")
    mfma = (f"# Matrix-core utilisation and clock, {tag}\n\ncommands (repository root, one MI355X):\n{cmds}\n\n"
            f"{header}\nPer dispatch: cycles = GRBM_GUI_ACTIVE / {XCDS} (one XCD's share), GHz = cycles / duration,\n"
            f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x cycles), CU busy = SQ_BUSY_CU_CYCLES / "
            f"({CUS} x cycles); medians per (kernel, workgroups).\n\n"
            f"| kernel | workgroups | dispatches | duration us | GHz | MFMA busy | CU busy |\n|---|---|---|---|---|---|---|\n"
            + "\n".join(mrows) + "\n")
    with open(os.path.join(args.summary_dir, f"chain_kernels_{tag}_mfma.md"), "w") as fh:
        fh.write(mfma)

    # ---- traffic
    def calib(name, counter):
        d = _counters(_find(raw, name, "counter_collection.csv"))
        vals = [c[counter] for k, wg, dur, c in d.values() if "copyBuffer" in k]
        if not vals:
            raise SystemExit(f"no copy dispatch in the {name} run")
        return COPY_MIB * 1024 / statistics.mean(vals)
    ff, fw = calib("cfetch", "FETCH_SIZE"), calib("cwrite", "WRITE_SIZE")
    fe = _chain_rows(_counters(_find(raw, "fetch", "counter_collection.csv")))
    wr = _chain_rows(_counters(_find(raw, "write", "counter_collection.csv")))
    trows, pers_bytes, pers_dur = [], None, None
    for key in sorted(fe):
        if key not in wr:
            continue
        fk = statistics.mean(c["FETCH_SIZE"] for _, c in fe[key])
        wk = statistics.mean(c["WRITE_SIZE"] for _, c in wr[key])
        dur = statistics.median(d for d, _ in fe[key] + wr[key])
        b = (fk * ff + wk * fw) * 1024
        trows.append(f"| {key[0]} | {key[1]} | {len(fe[key])} | {fk:.0f} | {wk:.0f} | {b / 1e9:.4f} GB | "
                     f"{dur:.1f} | {b / (dur * 1e-6) / 1e9:.0f} |")
        if key[0].startswith("chain_persistent_kernel"):
            pers_bytes, pers_dur = b, dur
    alg = w.bytes(args.M)
    traffic = (f"# Memory-side traffic, {tag}\n\ncommands (repository root, one MI355X), one counter per run:\n{cmds}\n\n"
               f"{header}\nCalibration: a {COPY_MIB} MiB device copy reads and writes {COPY_MIB * 1024} KiB per dispatch:\n"
               f"    FETCH_SIZE factor {ff:.4f}, WRITE_SIZE factor {fw:.4f}\n"
               f"FETCH_SIZE / WRITE_SIZE count L2 <-> fabric traffic, Infinity Cache hits included, so the figure\n"
               f"bounds HBM traffic from above.  Durations are the profiled dispatches' medians (counter runs).\n\n"
               f"| kernel | workgroups | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes/launch (calibrated) | "
               f"duration us | GB/s |\n|---|---|---|---|---|---|---|---|\n" + "\n".join(trows) + "\n\n"
               f"Algorithmic bytes of one chain pass (weights once, X, Y, T written and read once): {alg / 1e9:.4f} GB"
               + (f"; the persistent kernel moves {pers_bytes / alg:.2f}x that across the L2 boundary" if pers_bytes else "")
               + ".\n\n"
               f"plan: {plan}\n" + (f"traffic_bytes_per_launch: {int(pers_bytes)}\n" if pers_bytes else ""))
    with open(os.path.join(args.summary_dir, f"chain_persistent_kernel_{tag}_traffic.md"), "w") as fh:
        fh.write(traffic)
    print(f"summaries written to {args.summary_dir}/ for {tag}", flush=True)


if __name__ == "__main__":
    main()
