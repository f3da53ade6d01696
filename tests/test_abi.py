"""The C-ABI library loads and exports every symbol that include/mlp_chain.h
declares; argument checks that need no GPU behave as documented."""
import ctypes
import os
import re

import pytest

from consumer_gemm_chain_amd import mlp_chain as mc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlp_chain.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlp_chain_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for s in ("mlp_chain_create", "mlp_chain_run", "mlp_chain_destroy", "mlp_chain_run_phase",
              "mlp_chain_status", "mlp_chain_last_error"):
        assert s in syms
    assert set(syms) == set(mc.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mc.LIB_PATH)
    for s in declared_symbols():
        assert hasattr(lib, s), s


@pytest.mark.parametrize("args,needle", [
    ((0, 512, 512, 1, 0, 2), "sizes"),
    ((4, 500, 512, 1, 0, 2), "multiples of 8"),
    ((4, 512, 100, 1, 0, 2), "multiples of 8"),
    ((4, 512, 512, 3, 0, 2), "activation"),
    ((4, 512, 512, 1, 2, 2), "dtype"),
    ((4, 512, 512, 1, 0, 3), "policy"),
    ((4, 512, 512, -1, 0, 2), "activation"),
])
def test_create_rejects_bad_arguments(args, needle):
    lib = mc.load_library()
    assert not lib.mlp_chain_create(*args)
    assert needle in mc.mlp_chain_last_error()


def test_null_handle_entry_points():
    lib = mc.load_library()
    assert lib.mlp_chain_run(None, None, None, None, None, None) == mc.MLP_EINVAL
    assert lib.mlp_chain_run_phase(None, 1, None, None, None, None, None) == mc.MLP_EINVAL
    assert lib.mlp_chain_status(None) == mc.MLP_EINVAL
    assert lib.mlp_chain_destroy(None) == mc.MLP_OK
    assert lib.mlp_chain_debug_set_spin_limit(None, 5) == mc.MLP_EINVAL
    assert lib.mlp_chain_debug_skip_producer(None, 0) == mc.MLP_EINVAL
    assert lib.mlp_chain_debug_set_config(None, 0) == mc.MLP_EINVAL
    assert lib.mlp_chain_debug_set_split(None, 0, 0) == mc.MLP_EINVAL
    assert lib.mlp_chain_debug_set_grid(None, 0) == mc.MLP_EINVAL
    assert lib.mlp_chain_debug_set_order(None, 0) == mc.MLP_EINVAL
    assert lib.mlp_chain_set_weight_ld(None, 4096, 4096) == mc.MLP_EINVAL
    arr = (ctypes.c_int64 * 16)()
    assert lib.mlp_chain_info(None, arr, 16) == mc.MLP_EINVAL


def test_binding_raises_with_message():
    with pytest.raises(mc.MlpChainError) as e:
        mc.mlp_chain_create(4, 512, 100, mc.MLP_ACT_GELU_TANH, mc.MLP_DTYPE_F16, mc.MLP_POLICY_TILE_SYNC)
    assert "multiples of 8" in str(e.value)


@pytest.mark.parametrize("H,I,act", [(12288, 6144, "gelu_tanh"), (8192, 2752, "swiglu"), (8192, 3584, "swiglu"),
                                     (8192, 8192, "none"), (512, 2048, "gelu_tanh"), (200, 328, "swiglu"),
                                     (64, 64, "none")])
def test_preferred_weight_strides_cycle_line_classes(H, I, act):
    """mlp_chain_weight_ld (host only): the smallest row strides at least as
    wide as the rows whose byte length is an odd number of 128-byte lines,
    so the rows of a column panel visit all eight line classes."""
    g = 2 if act == "swiglu" else 1
    ld1, ld2 = mc.mlp_chain_weight_ld(H, I, mc.ACTS[act])
    for ld, n in ((ld1, g * I), (ld2, H)):
        assert n <= ld < n + 128 and ld % 8 == 0
        assert (ld * 2) % 256 == 128                      # odd number of 128-byte lines
        assert sorted({(r * ld * 2 // 128) % 8 for r in range(8)}) == list(range(8))
        assert all((m * 2) % 256 != 128 for m in range(n, ld, 8))   # the smallest such stride


def test_preferred_weight_strides_reject_bad_sizes():
    lib = mc.load_library()
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    assert lib.mlp_chain_weight_ld(500, 512, 1, ctypes.byref(a), ctypes.byref(b)) == mc.MLP_EINVAL
    assert lib.mlp_chain_weight_ld(512, 512, 3, ctypes.byref(a), ctypes.byref(b)) == mc.MLP_EINVAL
    assert lib.mlp_chain_weight_ld(512, 512, 1, None, ctypes.byref(b)) == mc.MLP_EINVAL
