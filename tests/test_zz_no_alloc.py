"""The entry point that allocates nothing (mlp_chain_run_noalloc), through
the C ABI: its output equals mlp_chain_run's bit for bit (same plan, same K
split), on two calls in a row, the second with a smaller input, for every
policy; a plan whose workspace exceeds the static scratch is refused with a
message."""
import ctypes

import numpy as np
import pytest

from consumer_gemm_chain_amd import gen
from consumer_gemm_chain_amd import mlp_chain as mc
from tests._helpers import empty_dev, from_dev, run_chain, to_dev

pytestmark = pytest.mark.gpu

# (M, H, I, act, dtype): a split-K case with a ragged inner width, then a
# smaller one
CASES = [(384, 2048, 1480, "gelu_tanh", "f16"), (70, 1024, 456, "gelu_tanh", "f16")]
SWIGLU = [(200, 1032, 776, "swiglu", "bf16"), (16, 512, 264, "swiglu", "bf16")]


def _noalloc(x, w1, w2, act, dtype, policy, status):
    import torch
    M, H = x.shape
    I = w2.shape[0]
    dx, dw1, dw2 = to_dev(x, dtype), to_dev(w1, dtype), to_dev(w2, dtype)
    out = empty_dev((M, H), dtype)
    out.fill_(float("nan"))
    status.fill_(7)
    s = torch.cuda.current_stream().cuda_stream
    mc.mlp_chain_run_noalloc(M, H, I, mc.ACTS[act], mc.DTYPES[dtype], mc.POLICIES[policy], dx.data_ptr(),
                             dw1.data_ptr(), dw2.data_ptr(), out.data_ptr(), status.data_ptr(), s)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return from_dev(out)


@pytest.mark.parametrize("cases", [CASES, SWIGLU], ids=["gelu_f16", "swiglu_bf16"])
@pytest.mark.parametrize("policy", ["stream_ordered", "row_sync", "tile_sync"])
def test_noalloc_matches_run_twice_then_smaller(cases, policy):
    import torch
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i, (M, H, I, act, dtype) in enumerate(cases):
        x, w1, w2 = gen.random_case(M, H, I, act, dtype, seed=50 + i, w_std=1.0 / np.sqrt(H))
        print(f"noalloc case M={M} H={H} I={I} act={act} dtype={dtype} policy={policy}", flush=True)
        ref = run_chain(x, w1, w2, act, dtype, policy)
        for rep in range(2):
            y = _noalloc(x, w1, w2, act, dtype, policy, status)
            assert np.array_equal(y, ref), (M, H, I, policy, rep)


def test_noalloc_planned_split_matches_run():
    """A weight-streaming shape whose plan splits K in both GEMMs (fp32
    partials and split counters in the scratch)."""
    import torch
    M, H, I, act, dtype = 16, 8192, 4096, "gelu_tanh", "f16"
    x, w1, w2 = gen.random_case(M, H, I, act, dtype, seed=61, w_std=1.0 / np.sqrt(H))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with mc.MlpChain(M, H, I, act, dtype, "tile_sync") as ch:
        info = ch.info()
        assert info["S1"] > 1 and info["S2"] > 1
    for pol in ("stream_ordered", "tile_sync"):
        ref = run_chain(x, w1, w2, act, dtype, pol)
        assert np.array_equal(_noalloc(x, w1, w2, act, dtype, pol, status), ref)


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    import torch
    lib = mc.load_library()
    n = 8192
    # full-size operands, so that nothing could read out of bounds even if the
    # call were (wrongly) accepted
    x, w1, w2, out = (torch.zeros((n, n), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    s = torch.cuda.current_stream().cuda_stream
    # the 8192^3 chain's intermediate alone is 128 MiB
    rc = lib.mlp_chain_run_noalloc(n, n, n, mc.MLP_ACT_NONE, mc.MLP_DTYPE_BF16, mc.MLP_POLICY_TILE_SYNC,
                                   x.data_ptr(), w1.data_ptr(), w2.data_ptr(), out.data_ptr(), None, s)
    assert rc == mc.MLP_EINVAL and "static scratch" in mc.mlp_chain_last_error()
    rc = lib.mlp_chain_run_noalloc(64, 512, 512, mc.MLP_ACT_NONE, mc.MLP_DTYPE_BF16, mc.MLP_POLICY_TILE_SYNC,
                                   x.data_ptr() + 2, w1.data_ptr(), w2.data_ptr(), out.data_ptr(), None, s)
    assert rc == mc.MLP_EINVAL and "aligned" in mc.mlp_chain_last_error()
    torch.cuda.synchronize()
