// chain_launch.h -- internal interface between the C ABI (chain_api.cpp) and
// the kernel launchers (chain_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "chain_device.hpp"

enum { LAUNCH_GEMM1 = 1, LAUNCH_GEMM2 = 2, LAUNCH_ROW = 3, LAUNCH_TILE = 4, LAUNCH_LAYERS_ROW = 5,
       LAUNCH_LAYERS_TILE = 6 };

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

// Resident workgroups per CU of the persistent kernel for a configuration
// (the multi-layer kernel when layers > 1).
hipError_t mlpc_persistent_occupancy(int cfg, int dtype, int policy, int layers, int* per_cu);

// The static device scratch of the entry point that allocates nothing
// (chain_scratch.hip): 128 MiB per device.
#define MLPC_SCRATCH_BYTES ((size_t)128 << 20)

// Address of `device`'s copy of the scratch (looked up once per device; the
// device must be current).
hipError_t mlpc_scratch_address(int device, void** ptr);

// Enqueue a kernel that zeroes `bytes` (a multiple of 16) at the 16-byte
// aligned device address p, and *status if non-null (no memset node, so the
// call may be captured into a graph).
hipError_t mlpc_zero_words(void* p, size_t bytes, uint32_t* status, hipStream_t s);

// The hand-off litmus kernel (chain_litmus.hip): `rounds` rounds of 256
// workgroups; data >= rounds x 1 MiB, flags >= rounds x 256 words and
// result >= 8 words, all zeroed by the caller.
hipError_t mlpc_litmus(void* data, size_t data_bytes, void* flags, size_t flag_bytes, void* result, int rounds,
                       int half_lines, int agent, uint32_t spin_limit, hipStream_t s);
