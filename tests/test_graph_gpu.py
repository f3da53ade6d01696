"""Fused runs captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A fused run keeps its epoch on the device, so its launch carries nothing
that changes between runs.  Every replay -- with direct runs of the same
handle, runs on other inputs and host synchronizations in between -- must
give the direct run's bits, which agree with the oracle and with the
stream-ordered kernels, and must advance the device's epoch by one."""
import numpy as np
import pytest

from consumer_gemm_chain_amd import gen
from consumer_gemm_chain_amd import mlp_chain as mc
from tests._helpers import check_against_oracle, empty_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("policy", ["row_sync", "tile_sync"])
@pytest.mark.parametrize("act,split", [("gelu_tanh", (1, 1)), ("gelu_tanh", (3, 2)), ("swiglu", (2, 3))])
def test_fused_graph_replays_match_direct_runs_and_oracle(oracle_mod, policy, act, split):
    import torch
    M, H, I, dtype = 200, 1024, 640, "f16"
    x, w1, w2 = gen.random_case(M, H, I, act, dtype, 7, w_std=1.0 / np.sqrt(H))
    decoy = np.ascontiguousarray(x[::-1])
    y_ref = oracle_mod.mlp_chain(x, w1, w2, act, dtype)
    dx, dd, dw1, dw2 = to_dev(x, dtype), to_dev(decoy, dtype), to_dev(w1, dtype), to_dev(w2, dtype)
    with mc.MlpChain(M, H, I, act, dtype, policy) as ch:
        ch.set_split(*split)
        ref_out = empty_dev((M, H), dtype)
        ch.run(dx, dw1, dw2, ref_out)
        torch.cuda.synchronize()
        ref = from_dev(ref_out)
        check_against_oracle(ref, y_ref, dtype, f"{policy} split {split}")
        with mc.MlpChain(M, H, I, act, dtype, "stream_ordered") as so:
            so.set_split(*split)
            so_out = empty_dev((M, H), dtype)
            so.run(dx, dw1, dw2, so_out)
            torch.cuda.synchronize()
            assert np.array_equal(ref, from_dev(so_out))
        out = empty_dev((M, H), dtype)
        g = _capture(lambda: ch.run(dx, dw1, dw2, out))
        e0 = ch.info()["epoch"]
        for i in range(6):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(out), ref), f"replay {i}"
            assert ch.info()["epoch"] == e0 + 2 * i + 1
            # direct work on the same handle between the replays: a run on
            # other inputs (a stale intermediate would show in the next replay)
            other = empty_dev((M, H), dtype)
            ch.run(dd, dw1, dw2, other)
            torch.cuda.synchronize()
            assert not np.array_equal(from_dev(other), ref)
        assert ch.status() == mc.MLP_OK


@pytest.mark.parametrize("policy", ["row_sync", "tile_sync"])
def test_fused_layers_graph_replays(oracle_mod, policy):
    """Two MLP layers (four dependent GEMMs) in one persistent kernel,
    captured and replayed back to back, ten replays in one graph launch
    sequence, then checked against the oracle's composition."""
    import torch
    L, M, H, I, act, dtype = 2, 96, 512, 384, "gelu_tanh", "bf16"
    x = gen.normal_bits((M, H), 31, 1.0, dtype)
    w1s = [gen.normal_bits((H, I), 40 + l, 1.0 / np.sqrt(H), dtype) for l in range(L)]
    w2s = [gen.normal_bits((I, H), 50 + l, 1.0 / np.sqrt(I), dtype) for l in range(L)]
    y_ref = oracle_mod.mlp_layers(x, w1s, w2s, act, dtype)
    dx = to_dev(x, dtype)
    dw1 = [to_dev(w, dtype) for w in w1s]
    dw2 = [to_dev(w, dtype) for w in w2s]
    with mc.MlpChain(M, H, I, act, dtype, policy, layers=L) as ch:
        direct = empty_dev((M, H), dtype)
        ch.run_layers(dx, dw1, dw2, direct)
        torch.cuda.synchronize()
        ref = from_dev(direct)
        check_against_oracle(ref, y_ref, dtype, f"{policy} layers")
        out = empty_dev((M, H), dtype)
        g = _capture(lambda: ch.run_layers(dx, dw1, dw2, out))
        e0 = ch.info()["epoch"]
        out.fill_(float("nan"))
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(out), ref)
        assert ch.info()["epoch"] == e0 + 10
        assert ch.status() == mc.MLP_OK
