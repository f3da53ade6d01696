// chain_launch.h -- internal interface between the C ABI (chain_api.cpp) and
// the kernel launchers (chain_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "chain_device.hpp"

enum { LAUNCH_GEMM1 = 1, LAUNCH_GEMM2 = 2, LAUNCH_ROW = 3, LAUNCH_TILE = 4 };

struct CfgInfo {
    int id;
    int BM, BN, BK, NT;   // BN: weight columns per tile (SwiGLU producers: BN/2 output columns)
    int lds;              // LDS bytes of the ring per workgroup
};

int mlpc_num_configs();
CfgInfo mlpc_config_info(int id);

// Launch one kernel of the chain.  `what` is LAUNCH_GEMM1 (grid a.T1),
// LAUNCH_GEMM2 (grid a.T2) or a persistent kernel (grid `grid`).
hipError_t mlpc_launch(const mlpc::ChainArgs& a, int cfg, int dtype, int what, int grid, hipStream_t s);

// Resident workgroups per CU of the persistent kernel for a configuration.
hipError_t mlpc_persistent_occupancy(int cfg, int dtype, int policy, int* per_cu);
