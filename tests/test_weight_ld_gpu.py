"""Weights with padded rows (mlp_chain_set_weight_ld): every policy reads
only the g I (W1) and H (W2) columns of each row, whatever the stride, so a
run on padded copies -- the padding filled with NaN -- gives the dense
run's bits, and both agree with the oracle."""
import numpy as np
import pytest

from consumer_gemm_chain_amd import gen
from consumer_gemm_chain_amd import mlp_chain as mc
from tests._helpers import POLICIES, check_against_oracle, empty_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _padded(t, ld):
    import torch
    p = torch.full((t.shape[0], ld), float("nan"), dtype=t.dtype, device=t.device)
    p[:, :t.shape[1]] = t
    return p[:, :t.shape[1]]


def _run(M, H, I, act, dtype, policy, x, w1, w2, ld=None, split=None):
    import torch
    with mc.MlpChain(M, H, I, act, dtype, policy) as ch:
        if split is not None:
            ch.set_split(*split)
        if ld is not None:
            ch.set_weight_ld(*ld)
        out = empty_dev((M, H), dtype)
        ch.run(x, w1, w2, out)
        torch.cuda.synchronize()
        assert ch.status() == mc.MLP_OK
        return from_dev(out)


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("act,dtype,split", [("gelu_tanh", "f16", None), ("swiglu", "bf16", None),
                                             ("gelu_tanh", "f16", (3, 2)), ("swiglu", "bf16", (2, 3))])
@pytest.mark.parametrize("which", ["preferred", "wide"])
def test_padded_weights_match_dense_and_oracle(oracle_mod, policy, act, dtype, split, which):
    M, H, I = 200, 1024, 648
    x, w1, w2 = gen.random_case(M, H, I, act, dtype, 11, w_std=1.0 / np.sqrt(H))
    y_ref = oracle_mod.mlp_chain(x, w1, w2, act, dtype)
    dx, dw1, dw2 = to_dev(x, dtype), to_dev(w1, dtype), to_dev(w2, dtype)
    g = 2 if act == "swiglu" else 1
    ld = mc.mlp_chain_weight_ld(H, I, mc.ACTS[act]) if which == "preferred" else (g * I + 520, H + 1000)
    assert ld[0] > g * I and ld[1] > H
    dense = _run(M, H, I, act, dtype, policy, dx, dw1, dw2, split=split)
    padded = _run(M, H, I, act, dtype, policy, dx, _padded(dw1, ld[0]), _padded(dw2, ld[1]), ld=ld, split=split)
    assert np.array_equal(padded, dense)
    check_against_oracle(padded, y_ref, dtype, f"{policy} padded {ld}")


@pytest.mark.parametrize("policy", POLICIES)
def test_padded_weights_in_a_layer_chain(policy):
    """Two layers, every layer's weights with the same padded strides: the
    same bits as the dense layer chain."""
    import torch
    L, M, H, I, act, dtype = 2, 96, 512, 384, "gelu_tanh", "f16"
    x = to_dev(gen.normal_bits((M, H), 5, 1.0, dtype), dtype)
    w1s = [to_dev(gen.normal_bits((H, I), 60 + l, 1.0 / np.sqrt(H), dtype), dtype) for l in range(L)]
    w2s = [to_dev(gen.normal_bits((I, H), 70 + l, 1.0 / np.sqrt(I), dtype), dtype) for l in range(L)]
    ld = mc.mlp_chain_weight_ld(H, I, mc.ACTS[act])
    outs = []
    for pad in (False, True):
        with mc.MlpChain(M, H, I, act, dtype, policy, layers=L) as ch:
            a1, a2 = w1s, w2s
            if pad:
                ch.set_weight_ld(*ld)
                a1 = [_padded(w, ld[0]) for w in w1s]
                a2 = [_padded(w, ld[1]) for w in w2s]
            out = empty_dev((M, H), dtype)
            ch.run_layers(x, a1, a2, out)
            torch.cuda.synchronize()
            assert ch.status() == mc.MLP_OK
            outs.append(from_dev(out))
    assert np.array_equal(outs[0], outs[1])


def test_weight_strides_are_checked():
    with mc.MlpChain(64, 512, 384, "swiglu", "f16", "tile_sync") as ch:
        for bad in ((767, 512), (768, 504), (772, 512), (768, 516), (1 << 25, 512)):
            with pytest.raises(mc.MlpChainError) as e:
                ch.set_weight_ld(*bad)
            assert "strides" in str(e.value)
        ch.set_weight_ld(832, 576)
        w1 = empty_dev((512, 768), "f16")             # dense rows, but the handle expects 832
        with pytest.raises(ValueError, match="row stride 832"):
            ch.run(empty_dev((64, 512), "f16"), w1, empty_dev((384, 512), "f16"), empty_dev((64, 512), "f16"))
