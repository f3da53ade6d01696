"""MI355X-native tile-synchronized MLP GEMM chain.

The compute path is the HIP library ``lib/libmlp_chain.so`` (built from
``csrc/`` for gfx950) behind the C ABI in ``include/mlp_chain.h``;
``mlp_chain`` is its ctypes binding and ``gen`` the seeded input
generator.  Importing the package does not load the library; the first
binding call does, and fails loudly if it has not been built.
"""
from .mlp_chain import (  # noqa: F401
    ACTS, DTYPES, POLICIES, MLP_OK, MLP_EINVAL, MLP_ENOMEM, MLP_EHIP, MLP_ETIMEOUT,
    MlpChain, MlpChainError, load_library,
    mlp_chain_create, mlp_chain_run, mlp_chain_destroy, mlp_chain_run_phase,
    mlp_chain_status, mlp_chain_last_error, mlp_chain_info,
    mlp_chain_debug_set_spin_limit, mlp_chain_debug_skip_producer, mlp_chain_debug_set_config,
    mlp_chain_debug_read_intermediate, mlp_chain_debug_set_split, mlp_chain_debug_set_trace,
)
