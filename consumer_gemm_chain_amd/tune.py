"""Per-shape plan tuner: measures tile configurations x K splits on the GPU
and writes the table the planner reads (csrc/tuned_plans.inc).

    python -m consumer_gemm_chain_amd.tune [--workloads 0,1,2,3,4] [--M 1,16] [--out PATH]

The pages' system tunes itself per GPU generation (FLUX summary card,
Interesting ideas: auto-tuned kernels); here each benchmarked shape (the
workloads' M lists) gets a measured plan instead of the planner's rules.
One constraint shapes the search: every policy of a shape must use the same
K split, because the split (not the tile shape) fixes the summation order,
and the fused policies must stay bit-identical to the stream-ordered pair.
So, per shape:
  1. every candidate split (S1, S2) is timed with every candidate tile
     configuration in each policy (event medians, hot);
  2. the split is the one whose best tile_sync time is lowest, decided
     among the three best by a longer re-timing, hot and with the Infinity
     Cache flushed by a 512 MB read (the mean of the two medians);
  3. each policy then takes its fastest configuration under that split,
     its candidates re-timed in alternating rounds.
The output is one MLPC_TUNED(M, H, I, act, cus, S1, S2, config_stream,
config_row, config_tile) line per shape, with the measured times as a
comment.  The planner uses a line only for the exact (M, H, I, act) and CU
count it was measured on and falls back to its rules elsewhere.
"""
from __future__ import annotations

import argparse
import datetime
import os
import sys
import time

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

OUT = os.path.join(PKG, "csrc", "tuned_plans.inc")
POLICIES = ("stream_ordered", "row_sync", "tile_sync")
MIN_SLABS = 8            # shortest K part considered (slabs of 64)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def candidate_configs(M):
    if M <= 16:
        return (0, 4, 9)
    if M <= 128:
        return (0, 4, 3, 10)
    if M <= 512:
        return (4, 3, 8, 10)
    return (3, 7, 8)


def candidate_splits(H, I):
    # (5 and 7 matter where a tile count such as LLaMA-65's 43 column tiles
    # makes 4 or 6 parts per tile leave CUs idle or spill into a second wave)
    n1, n2 = (H + 63) // 64, (I + 63) // 64
    s1s = [s for s in (1, 2, 3, 4, 5, 6, 7, 8) if s == 1 or n1 // s >= MIN_SLABS]
    s2s = [s for s in (1, 2, 3, 4, 5) if s == 1 or n2 // s >= MIN_SLABS]
    return [(a, b) for a in s1s for b in s2s]


def event_us(fn, n, stream, flush=None):
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
    return float(np.median(ts))


def time_plan(dev, w, M, policy, cfg, split, reps, stream, flush=None):
    import torch
    from consumer_gemm_chain_amd.mlp_chain import MlpChain
    x, w1, w2, out = dev
    with MlpChain(M, w.H, w.I, w.act, w.dtype, policy) as ch:
        ch.set_weight_ld(w1.stride(0), w2.stride(0))
        ch.set_config(cfg)
        ch.set_split(*split)
        for _ in range(2):
            ch.run(x[:M], w1, w2, out[:M])
        torch.cuda.synchronize()
        t = event_us(lambda: ch.run(x[:M], w1, w2, out[:M]), reps, stream, flush)
        if ch.status() != 0:
            raise RuntimeError(f"watchdog fired: {w.name} M={M} {policy} config {cfg} split {split}")
    return t


def tune_shape(dev, w, M, stream, flush_buf, cus):
    import torch
    cfgs = candidate_configs(M)
    splits = candidate_splits(w.H, w.I)
    reps = 12 if M <= 1024 else 6
    times = {}
    for split in splits:
        for pol in POLICIES:
            for cfg in cfgs:
                times[(split, pol, cfg)] = time_plan(dev, w, M, pol, cfg, split, reps, stream)
    best_tile = {s: min(times[(s, "tile_sync", c)] for c in cfgs) for s in splits}
    top = sorted(splits, key=lambda s: best_tile[s])[:3]
    # a read of 512 MB leaves the Infinity Cache holding clean lines and none
    # of the weights; a written flush would leave dirty lines whose write-back
    # overlaps the timed run
    flat = flush_buf.view(torch.float32)
    flush = lambda: flat.sum()  # noqa: E731
    score = {}
    for s in top:
        c = min(cfgs, key=lambda c: times[(s, "tile_sync", c)])
        hot = time_plan(dev, w, M, "tile_sync", c, s, 3 * reps, stream)
        cold = time_plan(dev, w, M, "tile_sync", c, s, max(4, reps), stream, flush)
        score[s] = (hot + cold) / 2
    split = min(top, key=lambda s: score[s])
    # each policy's configuration under that split: the candidates re-timed in
    # alternating rounds (the clock drifts with power and temperature, so
    # timings taken one after another favour whichever ran first)
    pick = {}
    for pol in POLICIES:
        rounds = {c: [] for c in cfgs}
        for _ in range(3):
            for c in cfgs:
                rounds[c].append(time_plan(dev, w, M, pol, c, split, reps, stream))
        for c in cfgs:
            times[(split, pol, c)] = float(np.median(rounds[c]))
        pick[pol] = min(cfgs, key=lambda c: times[(split, pol, c)])
    best_so = min((times[(s, "stream_ordered", c)], s, c) for s in splits for c in cfgs)
    entry = (M, w.H, w.I, {"none": 0, "gelu_tanh": 1, "swiglu": 2}[w.act], cus, split[0], split[1],
             pick["stream_ordered"], pick["row_sync"], pick["tile_sync"])
    note = (f"{w.name} M={M}: tile_sync {times[(split, 'tile_sync', pick['tile_sync'])]:.1f} us, "
            f"row_sync {times[(split, 'row_sync', pick['row_sync'])]:.1f} us, same-split pair "
            f"{times[(split, 'stream_ordered', pick['stream_ordered'])]:.1f} us; fastest pair of any split "
            f"{best_so[0]:.1f} us (config {best_so[2]}, split {best_so[1][0]},{best_so[1][1]})")
    log(note)
    return entry, note


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workloads", default="0,1,2,3,4")
    ap.add_argument("--M", default="", help="only these M of each workload (default: all of its M)")
    ap.add_argument("--out", default=OUT)
    args = ap.parse_args()
    only_m = {int(v) for v in args.M.split(",") if v.strip()}

    import torch
    from consumer_gemm_chain_amd import gen
    from consumer_gemm_chain_amd import mlp_chain as mc
    from consumer_gemm_chain_amd.tensors import to_dev, to_dev_rows
    mc.load_library()
    assert torch.cuda.is_available(), "the tuner measures on a GPU"
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    stream = torch.cuda.current_stream()
    flush_buf = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    lines = []
    t0 = time.time()
    for wl in (int(v) for v in args.workloads.split(",") if v.strip()):
        w = gen.WORKLOADS[wl]
        w1, w2 = gen.weights(w)
        x = gen.x_rows(w, w.max_M)
        # the weights in the row strides the library prefers (as the bench lays them out)
        ld1, ld2 = mc.mlp_chain_weight_ld(w.H, w.I, mc.ACTS[w.act])
        dev = (to_dev(x, w.dtype), to_dev_rows(w1, w.dtype, ld1), to_dev_rows(w2, w.dtype, ld2),
               torch.empty((w.max_M, w.H), dtype=torch.float16 if w.dtype == "f16" else torch.bfloat16,
                           device="cuda"))
        for M in w.Ms:
            if only_m and M not in only_m:
                continue
            entry, note = tune_shape(dev, w, M, stream, flush_buf, cus)
            lines.append(f"// {note}\nMLPC_TUNED({', '.join(str(v) for v in entry)})")
        del dev
        torch.cuda.empty_cache()
    head = (f"// Tuned plans: MLPC_TUNED(M, H, I, act, cus, S1, S2, config stream_ordered, config row_sync,\n"
            f"// config tile_sync).  Written by `python -m consumer_gemm_chain_amd.tune` on {props.name} ({cus} CUs),\n"
            f"// {datetime.date.today().isoformat()}, in {time.time() - t0:.0f} s; event medians, hot.\n")
    with open(args.out, "w") as fh:
        fh.write(head + "\n".join(lines) + "\n")
    log(f"wrote {len(lines)} plans to {args.out}")


if __name__ == "__main__":
    main()
