// chain_dispatch.cpp -- table of the per-configuration launchers (each
// configuration's kernels live in their own object, built from
// chain_kernels.hip with -DMLPC_CFG=<id>).
#include "chain_configs.h"
#include "chain_launch.h"

#define MLPC_DECL(id, ...)                                                                         \
    hipError_t mlpc_launch_cfg##id(const mlpc::ChainArgs&, int, int, int, hipStream_t);            \
    hipError_t mlpc_occupancy_cfg##id(int, int, int, int*);                                         \
    CfgInfo mlpc_info_cfg##id();
MLPC_CONFIGS(MLPC_DECL)
#undef MLPC_DECL

int mlpc_num_configs() { return MLPC_NUM_CONFIGS; }

CfgInfo mlpc_config_info(int id) {
#define MLPC_CASE(n, ...) \
    case n: return mlpc_info_cfg##n();
    switch (id) { MLPC_CONFIGS(MLPC_CASE) default: return CfgInfo{-1, 0, 0, 0, 0, 0}; }
#undef MLPC_CASE
}

hipError_t mlpc_launch(const mlpc::ChainArgs& a, int cfg, int dtype, int what, int grid, hipStream_t s) {
#define MLPC_CASE(n, ...) \
    case n: return mlpc_launch_cfg##n(a, dtype, what, grid, s);
    switch (cfg) { MLPC_CONFIGS(MLPC_CASE) default: return hipErrorInvalidValue; }
#undef MLPC_CASE
}

hipError_t mlpc_persistent_occupancy(int cfg, int dtype, int policy, int layers, int* per_cu) {
#define MLPC_CASE(n, ...) \
    case n: return mlpc_occupancy_cfg##n(dtype, policy, layers, per_cu);
    switch (cfg) { MLPC_CONFIGS(MLPC_CASE) default: return hipErrorInvalidValue; }
#undef MLPC_CASE
}
