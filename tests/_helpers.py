"""Shared helpers of the GPU tests: device transfer of bit patterns, runs
through the C ABI, and the acceptance checks against the oracle."""
from __future__ import annotations

import numpy as np

from consumer_gemm_chain_amd import gen
from consumer_gemm_chain_amd.mlp_chain import MLP_OK, MlpChain
from consumer_gemm_chain_amd.tensors import empty_dev, from_dev, to_dev, torch_dtype  # noqa: F401

POLICIES = ("stream_ordered", "row_sync", "tile_sync")

# elementwise acceptance |gpu - oracle| <= ATOL + RTOL * |oracle|
TOL = {"f16": (1e-2, 1e-2), "bf16": (2e-2, 2e-2)}
# supplementary normwise bound ||gpu - oracle||_F / ||oracle||_F
NORMWISE = {"f16": 2.0 ** -8, "bf16": 2.0 ** -5}


def run_chain(x, w1, w2, act, dtype, policy, cfg=None, reps=1, dev=None, chain=None):
    """Run the chain on the GPU through the C ABI and return Y bits.
    `dev` may hold already-transferred (x, w1, w2) tensors."""
    import torch
    M, H = x.shape
    I = w2.shape[0]
    dx, dw1, dw2 = dev if dev is not None else (to_dev(x, dtype), to_dev(w1, dtype), to_dev(w2, dtype))
    out = empty_dev((M, H), dtype)
    own = chain is None
    ch = chain or MlpChain(M, H, I, act, dtype, policy)
    try:
        if cfg is not None:
            ch.set_config(cfg)
        for _ in range(reps):
            ch.run(dx, dw1, dw2, out)
        torch.cuda.synchronize()
        st = ch.status()
        assert st == MLP_OK, f"device status {st}"
        return from_dev(out)
    finally:
        if own:
            ch.close()


def widen(bits, dtype):
    return gen.from_bits(bits, dtype).astype(np.float64)


def check_against_oracle(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str, what: str = ""):
    g, r = widen(y_gpu, dtype), widen(y_ref, dtype)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    atol, rtol = TOL[dtype]
    err = np.abs(g - r)
    lim = atol + rtol * np.abs(r)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{what}: {len(bad)} elements outside tolerance, first at {bad[0].tolist()}: "
                           f"gpu={g[tuple(bad[0])]} oracle={r[tuple(bad[0])]}")
    nrm = np.linalg.norm(r)
    if nrm > 0:
        rel = np.linalg.norm(g - r) / nrm
        assert rel <= NORMWISE[dtype], f"{what}: normwise error {rel:.3e} > {NORMWISE[dtype]:.3e}"
    else:
        assert np.all(g == 0)
    return float(np.max(err)) if err.size else 0.0
