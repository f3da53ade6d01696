"""GPU-side behaviour of the C ABI: argument errors, the phase entry point,
the watchdog path (forced from the host, so every kernel still exits
normally), and handle lifetime."""
import ctypes

import numpy as np
import pytest

from consumer_gemm_chain_amd import gen
from consumer_gemm_chain_amd import mlp_chain as mc
from tests._helpers import empty_dev, from_dev, run_chain, to_dev

pytestmark = pytest.mark.gpu


def _inputs(M=96, H=256, I=384, act="gelu_tanh", dtype="f16", seed=1):
    x, w1, w2 = gen.random_case(M, H, I, act, dtype, seed, w_std=1.0 / np.sqrt(H))
    return x, w1, w2, (to_dev(x, dtype), to_dev(w1, dtype), to_dev(w2, dtype))


def test_misaligned_and_null_pointers_rejected():
    import torch
    x, w1, w2, (dx, dw1, dw2) = _inputs()
    out = empty_dev((96, 256), "f16")
    lib = mc.load_library()
    h = mc.mlp_chain_create(96, 256, 384, mc.MLP_ACT_GELU_TANH, mc.MLP_DTYPE_F16, mc.MLP_POLICY_TILE_SYNC)
    try:
        s = torch.cuda.current_stream().cuda_stream
        rc = lib.mlp_chain_run(h, dx.data_ptr() + 2, dw1.data_ptr(), dw2.data_ptr(), out.data_ptr(), s)
        assert rc == mc.MLP_EINVAL and "aligned" in mc.mlp_chain_last_error()
        rc = lib.mlp_chain_run(h, dx.data_ptr(), None, dw2.data_ptr(), out.data_ptr(), s)
        assert rc == mc.MLP_EINVAL
        rc = lib.mlp_chain_run_phase(h, 3, dx.data_ptr(), dw1.data_ptr(), None, None, s)
        assert rc == mc.MLP_EINVAL
        assert mc.mlp_chain_status(h) == mc.MLP_OK
        info = mc.mlp_chain_info(h)
        assert info["epoch"] == 0          # rejected runs do not advance the epoch
        # tile-order hook: order bits 0..1 and XCD rows 1, 2, 4 or 8 in bits 4..7
        for bad in (-2, 4, 3 << 4, 5 << 4, 16 << 4):
            assert lib.mlp_chain_debug_set_order(h, bad) == mc.MLP_EINVAL, bad
        for good in (-1, 0, 3, 1 << 4, 2 | (8 << 4)):
            assert lib.mlp_chain_debug_set_order(h, good) == mc.MLP_OK, good
    finally:
        mc.mlp_chain_destroy(h)


@pytest.mark.parametrize("policy", ["stream_ordered", "tile_sync"])
def test_phases_compose_to_the_chain(policy):
    import torch
    x, w1, w2, dev = _inputs()
    ref = run_chain(x, w1, w2, "gelu_tanh", "f16", "stream_ordered", dev=dev)
    with mc.MlpChain(96, 256, 384, "gelu_tanh", "f16", policy) as ch:
        out = empty_dev((96, 256), "f16")
        ch.run_phase(1, x=dev[0], w1=dev[1])
        ch.run_phase(2, w2=dev[2], out=out)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(out), ref)


@pytest.mark.parametrize("policy", ["row_sync", "tile_sync"])
def test_watchdog_reports_timeout_and_recovers(policy):
    """Producer tile 0 is told (from the host) to skip its work and its
    release; the consumers that need it give up after a short spin limit,
    the handle reports MLP_ETIMEOUT, and the next run is correct again."""
    import torch
    x, w1, w2, dev = _inputs()
    ref = run_chain(x, w1, w2, "gelu_tanh", "f16", "stream_ordered", dev=dev)
    with mc.MlpChain(96, 256, 384, "gelu_tanh", "f16", policy) as ch:
        out = empty_dev((96, 256), "f16")
        ch.run(*dev, out)
        torch.cuda.synchronize()
        assert ch.status() == mc.MLP_OK
        ch.set_spin_limit(2000)
        ch.skip_producer(0)
        ch.run(*dev, out)
        torch.cuda.synchronize()
        assert ch.status() == mc.MLP_ETIMEOUT
        assert "gave up" in mc.mlp_chain_last_error()
        ch.skip_producer(-1)
        ch.set_spin_limit(0)
        out.fill_(0)
        ch.run(*dev, out)
        torch.cuda.synchronize()
        assert ch.status() == mc.MLP_OK
        assert np.array_equal(from_dev(out), ref)


def test_create_destroy_does_not_leak():
    import torch
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(30):
        h = mc.mlp_chain_create(2048, 4096, 4096, mc.MLP_ACT_SWIGLU, mc.MLP_DTYPE_BF16,
                                mc.MLP_POLICY_TILE_SYNC)
        mc.mlp_chain_destroy(h)
    free1, _ = torch.cuda.mem_get_info()
    assert free0 - free1 < 64 << 20


def test_info_reports_plan():
    with mc.MlpChain(4096, 8192, 3584, "swiglu", "bf16", "tile_sync") as ch:
        info = ch.info()
        assert info["cus"] >= 1 and info["grid"] >= 1 and info["wg_per_cu"] >= 1
        assert info["T1"] == info["Mt"] * info["N1t"] and info["T2"] == info["Mt"] * info["N2t"]
        assert info["grid"] <= info["wg_per_cu"] * info["cus"]
        assert info["S1"] == 1 and info["S2"] == 1          # enough tiles: no split
    with mc.MlpChain(1, 8192, 4096, "gelu_tanh", "f16", "tile_sync") as ch:
        info = ch.info()
        assert info["S1"] > 1 and info["S2"] > 1            # weight streaming: split K
        assert info["ksp1"] * info["S1"] >= 8192 // 64 and info["ksp2"] * info["S2"] >= 4096 // 64
        assert (info["S1"] - 1) * info["ksp1"] < 8192 // 64  # no empty part
        assert info["ksp1"] >= 24 and info["ksp2"] >= 24


def test_fused_split_plan_is_shared_by_every_policy():
    """Where GEMM1's unsplit tiles make between half a wave and one wave and
    each half keeps >= 96 K slabs (GPT-3 shard, M = 1024 and 2048), GEMM1 is
    split in two for every policy; each policy keeps its own tile shape."""
    cus = None
    for M in (1024, 2048):
        plans = {}
        for pol in ("stream_ordered", "row_sync", "tile_sync"):
            with mc.MlpChain(M, 12288, 6144, "gelu_tanh", "f16", pol) as ch:
                plans[pol] = ch.info()
                cus = plans[pol]["cus"]
        if cus != 256:
            pytest.skip(f"plan thresholds are for 256 CUs, this GPU has {cus}")
        for pol, info in plans.items():
            assert (info["S1"], info["S2"]) == (2, 1), (M, pol, info)
        fused = plans["tile_sync"]
        assert fused["BM"] == 256 and 128 < fused["T1"] <= 256, fused
        # the fused policies use the same tile shape (configurations 7 and 8
        # differ only in their LDS ring)
        assert (plans["row_sync"]["BM"], plans["row_sync"]["BN1"]) == (fused["BM"], fused["BN1"])
    # the LLaMA-65 shard (64-slab halves) keeps the unsplit plan at M = 2048
    with mc.MlpChain(2048, 8192, 2752, "swiglu", "f16", "tile_sync") as ch:
        assert ch.info()["S1"] == 1


@pytest.mark.parametrize("policy", ["row_sync", "tile_sync"])
def test_watchdog_with_split_producer(policy):
    """A skipped part of a split producer tile means the tile is never
    reduced or published: its consumers time out and the handle recovers."""
    import torch
    x, w1, w2, dev = _inputs(M=32, H=2048, I=1024)
    ref = run_chain(x, w1, w2, "gelu_tanh", "f16", "stream_ordered", dev=dev)
    with mc.MlpChain(32, 2048, 1024, "gelu_tanh", "f16", policy) as ch:
        ch.set_split(4, 2)
        out = empty_dev((32, 2048), "f16")
        ch.set_spin_limit(2000)
        ch.skip_producer(1)              # tile 0, part 1
        ch.run(*dev, out)
        torch.cuda.synchronize()
        assert ch.status() == mc.MLP_ETIMEOUT
        ch.skip_producer(-1)
        ch.set_spin_limit(0)
        ch.run(*dev, out)
        torch.cuda.synchronize()
        assert ch.status() == mc.MLP_OK
        # same split in a stream-ordered handle for the bitwise comparison
        with mc.MlpChain(32, 2048, 1024, "gelu_tanh", "f16", "stream_ordered") as so:
            so.set_split(4, 2)
            out2 = empty_dev((32, 2048), "f16")
            so.run(*dev, out2)
            torch.cuda.synchronize()
        assert np.array_equal(from_dev(out), from_dev(out2))


@pytest.mark.parametrize("split", [(1, 1), (3, 2)])
def test_stream_ordered_graph_replays_match_eager(oracle_mod, split):
    """The stream-ordered pair captured in a HIP graph (torch.cuda.CUDAGraph)
    and replayed: every replay -- with eager runs of the same handle and host
    synchronizations in between -- gives the eager result bit for bit, and
    that result agrees with the oracle.  With a K split this relies on the
    split-K arrival counters returning to zero after every execution."""
    import torch
    from tests._helpers import check_against_oracle
    M, H, I = 96, 1024, 640
    x, w1, w2, dev = _inputs(M=M, H=H, I=I)
    y_ref = oracle_mod.mlp_chain(x, w1, w2, "gelu_tanh", "f16")
    with mc.MlpChain(M, H, I, "gelu_tanh", "f16", "stream_ordered") as ch:
        ch.set_split(*split)
        ref_out = empty_dev((M, H), "f16")
        ch.run(*dev, ref_out)
        torch.cuda.synchronize()
        ref = from_dev(ref_out)
        check_against_oracle(ref, y_ref, "f16", f"graph split {split}")
        out = empty_dev((M, H), "f16")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            ch.run(*dev, out)                      # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ch.run(*dev, out)
        for i in range(5):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(out), ref), f"replay {i}"
            eager = empty_dev((M, H), "f16")
            ch.run(*dev, eager)                    # eager work between the replays
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(eager), ref), f"eager run after replay {i}"
        assert ch.status() == 0
