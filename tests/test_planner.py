"""The planner, on the host alone (mlp_chain_plan touches no device): the
K split is shared by every policy (the bit-exactness contract), every part
is non-empty and the tiles cover the matrices, and the documented rules pick
the configurations and splits they state for the five workloads."""
import itertools

import pytest

from consumer_gemm_chain_amd import gen
from consumer_gemm_chain_amd import mlp_chain as mc

CUS = 256
POLS = (mc.MLP_POLICY_STREAM_ORDERED, mc.MLP_POLICY_ROW_SYNC, mc.MLP_POLICY_TILE_SYNC)
MS = (1, 2, 15, 16, 17, 64, 100, 128, 256, 257, 512, 768, 1024, 1536, 2048, 4096, 8192)


def plan(M, H, I, act, policy, cus=CUS):
    """The rules' plan (the tuned table left out)."""
    return mc.mlp_chain_plan(M, H, I, mc.ACTS[act], policy, -cus)


def planned(M, H, I, act, policy, cus=CUS):
    """The plan create makes: a tuned plan where the table has one."""
    return mc.mlp_chain_plan(M, H, I, mc.ACTS[act], policy, cus)


def tuned_entries():
    import os
    import re
    path = os.path.join(os.path.dirname(mc.PKG), "consumer_gemm_chain_amd", "csrc", "tuned_plans.inc")
    text = re.sub(r"//[^\n]*", "", open(path).read())
    return [tuple(int(v) for v in m.split(",")) for m in re.findall(r"MLPC_TUNED\(([^)]*)\)", text)]


def cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("wl", range(len(gen.WORKLOADS)))
def test_split_shared_by_policies_and_parts_cover_k(wl):
    w = gen.WORKLOADS[wl]
    for M, cus, fn in itertools.product(MS, (CUS, 80, 304), (plan, planned)):
        plans = [fn(M, w.H, w.I, w.act, pol, cus) for pol in POLS]
        assert len({(p["S1"], p["S2"]) for p in plans}) == 1, (w.name, M, cus, plans)
        for p in plans:
            nks1, nks2 = cdiv(w.H, 64), cdiv(w.I, 64)
            for S, ksp, nks in ((p["S1"], p["ksp1"], nks1), (p["S2"], p["ksp2"], nks2)):
                assert S >= 1 and (S - 1) * ksp < nks <= S * ksp, (w.name, M, p)
            assert p["Mt"] * p["BM"] >= M and (p["Mt"] - 1) * p["BM"] < M
            assert p["N1t"] * p["BN1"] >= w.I and p["N2t"] * p["BN2"] >= w.H
            assert p["T1"] == p["Mt"] * p["N1t"] and p["T2"] == p["Mt"] * p["N2t"]
            assert p["BN1"] == (p["BN2"] // 2 if w.act == "swiglu" else p["BN2"])


def test_small_m_configurations():
    w = gen.WORKLOADS[1]                       # GPT-3 shard
    for M in (1, 16):
        for pol in POLS:
            p = plan(M, w.H, w.I, w.act, pol)
            assert (p["BM"], p["BN2"]) == (16, 64)
            assert p["S1"] * p["T1"] <= CUS and p["S1"] > 1     # weight streaming: split K
    p = plan(64, w.H, w.I, w.act, mc.MLP_POLICY_TILE_SYNC)
    assert (p["BM"], p["BN2"]) == (64, 128) and p["T1"] <= CUS and p["T2"] < CUS
    # LLaMA-65 at M = 256: GEMM2 would have exactly one wave of 64 x 128
    # tiles -- the 256-row tiles with a K split take over
    w = gen.WORKLOADS[2]
    for pol in POLS:
        p = plan(256, w.H, w.I, w.act, pol)
        assert p["BM"] == 256 and (p["S1"], p["S2"]) == (4, 1), p


@pytest.mark.parametrize("M,fused_tile,so_tile", [(1024, (256, 128), (256, 256)), (2048, (256, 256), (256, 128))])
def test_fused_split_of_gemm1_on_the_gpt3_shard(M, fused_tile, so_tile):
    """GEMM1's unsplit tiles make between half a wave and one wave and each
    half keeps >= 96 K slabs: GEMM1 is split in two for every policy; the
    fused policies take the configuration the rule names, the stream-ordered
    pair the one with the fewer wave-rounded slab steps for that split."""
    w = gen.WORKLOADS[1]
    fused = plan(M, w.H, w.I, w.act, mc.MLP_POLICY_TILE_SYNC)
    so = plan(M, w.H, w.I, w.act, mc.MLP_POLICY_STREAM_ORDERED)
    assert (fused["S1"], fused["S2"]) == (2, 1) == (so["S1"], so["S2"])
    assert (fused["BM"], fused["BN2"]) == fused_tile and (so["BM"], so["BN2"]) == so_tile
    assert CUS // 2 < fused["T1"] <= CUS
    assert fused["ksp1"] >= 96
    assert plan(M, w.H, w.I, w.act, mc.MLP_POLICY_ROW_SYNC)["config"] == fused["config"]


@pytest.mark.parametrize("wl", [2, 3, 4])
def test_no_fused_split_where_halves_are_short(wl):
    """H = 8192 (128 K slabs): halves of 64 slabs lost more to the fp32
    partials than they gained, so GEMM1 stays unsplit once it has enough
    tiles."""
    w = gen.WORKLOADS[wl]
    for M in (1024, 2048, 4096, 8192):
        if M < 2048 and w.act == "none":
            continue
        assert plan(M, w.H, w.I, w.act, mc.MLP_POLICY_TILE_SYNC)["S1"] == 1, (w.name, M)


def test_large_m_has_no_split_and_large_tiles():
    for wl, M in ((3, 8192), (4, 8192), (3, 4096)):
        w = gen.WORKLOADS[wl]
        for pol in POLS:
            p = plan(M, w.H, w.I, w.act, pol)
            assert (p["S1"], p["S2"]) == (1, 1)
            assert (p["BM"], p["BN2"]) == (256, 256), (w.name, M, pol, p)


@pytest.mark.parametrize("args", [
    (0, 512, 512, 1, 2, 256), (4, 500, 512, 1, 2, 256), (4, 512, 512, 3, 2, 256),
    (4, 512, 512, 1, 3, 256), (4, 512, 512, 1, 2, 4),
])
def test_plan_rejects_bad_arguments(args):
    import ctypes
    lib = mc.load_library()
    arr = (ctypes.c_int64 * 14)()
    assert lib.mlp_chain_plan(*args, arr, 14) == mc.MLP_EINVAL
    assert lib.mlp_chain_plan(64, 512, 512, 1, 2, 256, None, 13) == mc.MLP_EINVAL
    assert lib.mlp_chain_plan(64, 512, 512, 1, 2, 256, arr, 2) == mc.MLP_EINVAL


def test_tuned_table_entries_are_used_and_valid():
    """Every measured plan in the tuned table is what create would use for
    its exact shape and CU count (one split for every policy, each policy its
    measured configuration); other CU counts fall back to the rules."""
    from consumer_gemm_chain_amd import build as b
    ncfg = b.num_configs()
    acts = {v: k for k, v in mc.ACTS.items()}
    for (M, H, I, act, cus, s1, s2, c0, c1, c2) in tuned_entries():
        for pol, cfg in zip(POLS, (c0, c1, c2)):
            assert 0 <= cfg < ncfg
            p = planned(M, H, I, acts[act], pol, cus)
            assert p["tuned"] == 1 and (p["config"], p["S1"], p["S2"]) == (cfg, s1, s2), (M, H, I, pol, p)
            assert plan(M, H, I, acts[act], pol, cus)["tuned"] == 0
        assert planned(M, H, I, acts[act], POLS[0], cus + 8)["tuned"] == 0
