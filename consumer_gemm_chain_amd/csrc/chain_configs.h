// chain_configs.h -- the tile configurations the library is built with.
// X(id, BM, BN, WM, WN, NS, OCC): BM x BN tile, WM x WN waves, NS LDS
// stages, persistent-kernel register target OCC waves per SIMD.
#pragma once

#define MLPC_CONFIGS(X)                                                                        \
    X(0, 16, 64, 1, 2, 4, 2)     /* small M: narrow tiles, weight streaming */                \
    X(1, 64, 128, 2, 2, 2, 2)    /* medium M, two stages */                                   \
    X(2, 128, 128, 2, 2, 2, 2)   /* large M, two stages: two workgroups per CU */             \
    X(3, 256, 128, 2, 2, 2, 1)   /* 128x64 per wave, one wave per SIMD */                     \
    X(4, 128, 256, 2, 2, 2, 1)   /* 64x128 per wave, one wave per SIMD */                     \
    X(5, 16, 128, 1, 2, 4, 1)    /* small M, 16x64 per wave */                                \
    X(6, 128, 256, 2, 4, 2, 2)   /* eight waves of 64x64 */                                   \
    X(7, 256, 128, 4, 2, 2, 2)   /* eight waves of 64x64 */                                   \
    X(8, 128, 256, 2, 4, 3, 2)   /* eight waves of 64x64, three stages */                     \
    X(9, 256, 128, 4, 2, 3, 2)   /* large M: eight waves of 64x64, three stages, one WG per CU */ \
    X(10, 64, 128, 2, 2, 4, 1)   /* exp: weight streaming, three slabs in flight */           \
    X(11, 32, 128, 1, 2, 4, 1)   /* exp */                                                    \
    X(12, 16, 256, 1, 2, 4, 1)   /* exp: decode, 512-byte weight strips */

#define MLPC_COUNT_CFG(id, ...) +1
constexpr int MLPC_NUM_CONFIGS = 0 MLPC_CONFIGS(MLPC_COUNT_CFG);
