"""The synchronization under shifted timing: the test build of the library
(libmlp_chain_chaos.so, compiled with MLPC_CHAOS=1) pauses a pseudo-random
time of up to about 16 us before every tile or split part publishes.  Many
runs per handle, alternating two inputs, must each equal the stream-ordered
output of the normal build for their input, bit for bit: a consumer or a
reducing part that read before its producer published would see the other
input's values (left by the previous run) and differ."""
import ctypes

import numpy as np
import pytest

from consumer_gemm_chain_amd import gen
from consumer_gemm_chain_amd import mlp_chain as mc
from tests._helpers import empty_dev, from_dev, run_chain, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chaos():
    # torch's HIP runtime first (as everywhere else: the library is loaded
    # after torch has initialized the device)
    import torch
    torch.cuda.init()
    mc.load_library()
    return mc.load_chaos_library()


def _case(M, H, I, act, dtype, seed):
    return gen.random_case(M, H, I, act, dtype, seed, w_std=1.0 / np.sqrt(H))


@pytest.mark.parametrize("M,H,I,act,dtype,cfg,split", [
    (512, 1024, 1536, "gelu_tanh", "f16", 3, None),
    (300, 1032, 776, "swiglu", "bf16", 0, None),     # 32-column producer tiles (agent-scope hand-off)
    (40, 2048, 1088, "gelu_tanh", "f16", 4, (3, 2)),
    (600, 1024, 1024, "none", "bf16", 7, (2, 1)),
    (16, 2048, 1536, "gelu_tanh", "f16", 9, (4, 2)),
    (256, 1024, 704, "swiglu", "f16", 10, (2, 1)),
])
@pytest.mark.parametrize("policy", ["row_sync", "tile_sync"])
def test_chaos_repeated_runs(chaos, M, H, I, act, dtype, cfg, split, policy):
    import torch
    print(f"chaos {policy} M={M} H={H} I={I} act={act} dtype={dtype} cfg={cfg} split={split}", flush=True)
    xa, w1, w2 = _case(M, H, I, act, dtype, seed=M)
    xb = gen.normal_bits((M, H), M + 1, 1.0, dtype)
    dw1, dw2 = to_dev(w1, dtype), to_dev(w2, dtype)
    dxs = [to_dev(xa, dtype), to_dev(xb, dtype)]
    refs = []
    for dx, x in zip(dxs, (xa, xb)):
        with mc.MlpChain(M, H, I, act, dtype, "stream_ordered") as so:
            so.set_config(cfg)
            if split:
                so.set_split(*split)
            out = empty_dev((M, H), dtype)
            so.run(dx, dw1, dw2, out)
            torch.cuda.synchronize()
            refs.append(from_dev(out))
    assert not np.array_equal(refs[0], refs[1])
    h = chaos.mlp_chain_create(M, H, I, mc.ACTS[act], mc.DTYPES[dtype], mc.POLICIES[policy])
    assert h
    try:
        assert chaos.mlp_chain_debug_set_config(h, cfg) == mc.MLP_OK
        if split:
            assert chaos.mlp_chain_debug_set_split(h, *split) == mc.MLP_OK
        out = empty_dev((M, H), dtype)
        s = torch.cuda.current_stream().cuda_stream
        for i in range(64):
            out.fill_(float("nan"))
            assert chaos.mlp_chain_run(h, dxs[i % 2].data_ptr(), dw1.data_ptr(), dw2.data_ptr(), out.data_ptr(),
                                       s) == mc.MLP_OK
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(out), refs[i % 2]), (policy, i)
        assert chaos.mlp_chain_status(h) == mc.MLP_OK
    finally:
        chaos.mlp_chain_destroy(h)


@pytest.mark.parametrize("policy", ["row_sync", "tile_sync"])
def test_chaos_layers(chaos, policy):
    """Three layers in one persistent kernel under the pauses."""
    import torch
    M, H, I, L, act, dtype = 200, 520, 456, 3, "gelu_tanh", "f16"
    xs = [gen.normal_bits((M, H), 90 + i, 1.0, dtype) for i in range(2)]
    w1s = [gen.normal_bits((H, I), 95 + l, 1.0 / np.sqrt(H), dtype) for l in range(L)]
    w2s = [gen.normal_bits((I, H), 99 + l, 1.0 / np.sqrt(I), dtype) for l in range(L)]
    refs = []
    for x in xs:
        y = x
        for w1, w2 in zip(w1s, w2s):
            y = run_chain(y, w1, w2, act, dtype, "stream_ordered")
        refs.append(y)
    dxs = [to_dev(x, dtype) for x in xs]
    dw1 = [to_dev(w, dtype) for w in w1s]
    dw2 = [to_dev(w, dtype) for w in w2s]
    a1 = (ctypes.c_void_p * L)(*[w.data_ptr() for w in dw1])
    a2 = (ctypes.c_void_p * L)(*[w.data_ptr() for w in dw2])
    h = chaos.mlp_chain_create_layers(M, H, I, mc.ACTS[act], mc.DTYPES[dtype], mc.POLICIES[policy], L)
    assert h
    try:
        out = empty_dev((M, H), dtype)
        s = torch.cuda.current_stream().cuda_stream
        for i in range(16):
            out.fill_(float("nan"))
            assert chaos.mlp_chain_run_layers(h, dxs[i % 2].data_ptr(), a1, a2, out.data_ptr(), s) == mc.MLP_OK
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(out), refs[i % 2]), (policy, i)
        assert chaos.mlp_chain_status(h) == mc.MLP_OK
    finally:
        chaos.mlp_chain_destroy(h)
