// chain_configs.h -- the tile configurations the library is built with.
// X(id, BM, BN, WM, WN, NS, OCC, KS): BM x BN tile, WM x WN waves, NS LDS
// stages of KS K-elements each (64: a whole slab, 32: half a slab),
// persistent-kernel register target OCC waves per SIMD.
#pragma once

#define MLPC_CONFIGS(X)                                                                        \
    X(0, 16, 64, 1, 2, 4, 2, 64)     /* M <= 16: weight streaming, four stages */                 \
    X(1, 64, 128, 2, 2, 2, 2, 64)    /* measurements: two stages, up to three workgroups per CU */ \
    X(2, 128, 128, 2, 2, 2, 2, 64)   /* measurements: two stages, two workgroups per CU */         \
    X(3, 256, 128, 4, 2, 3, 2, 64)   /* M > 16 beyond one wave of 64x128 tiles: eight waves */      \
    X(4, 64, 128, 2, 2, 4, 1, 64)    /* M <= 256, one wave of tiles: four stages, one WG per CU */ \
    X(5, 256, 128, 2, 2, 3, 1, 64)   /* measurements: four waves of 128x64 */                     \
    X(6, 128, 256, 2, 4, 3, 2, 64)   /* measurements: eight waves of 64x64, 128 x 256 */          \
    X(7, 256, 256, 2, 4, 2, 2, 64)   /* large M once these tiles fill the GPU: eight waves of 128x64 */ \
    X(8, 256, 256, 2, 4, 4, 2, 32)   /* 256 x 256 on a ring of four half slabs: three in flight */ \
    X(9, 16, 128, 1, 2, 4, 1, 64)    /* M <= 16 SwiGLU: 64 output columns, whole 128-byte lines of T */ \
    X(10, 128, 128, 2, 4, 4, 1, 64)  /* mid M: eight waves of 64x32, four stages; a quarter of the partials of 256 x 128 */

#define MLPC_COUNT_CFG(id, ...) +1
constexpr int MLPC_NUM_CONFIGS = 0 MLPC_CONFIGS(MLPC_COUNT_CFG);
