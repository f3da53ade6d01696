// chain_configs.h -- the tile configurations the library is built with.
// X(id, BM, BN, WM, WN, NS, OCC): BM x BN tile, WM x WN waves, NS LDS
// stages, persistent-kernel register target OCC waves per SIMD.
#pragma once

#define MLPC_CONFIGS(X)                                                                        \
    X(0, 16, 64, 1, 2, 4, 4)     /* small M: narrow tiles, weight streaming */                \
    X(1, 64, 128, 2, 2, 2, 2)    /* medium M, two stages */                                   \
    X(2, 128, 128, 2, 2, 2, 2)   /* large M, two stages: two workgroups per CU */             \
    X(3, 128, 128, 2, 2, 3, 1)   /* large M, three stages, one workgroup per CU */            \
    X(4, 256, 128, 4, 2, 3, 2)   /* large M, 8 waves of 64x64 */

#define MLPC_COUNT_CFG(id, ...) +1
constexpr int MLPC_NUM_CONFIGS = 0 MLPC_CONFIGS(MLPC_COUNT_CFG);
