// chain_device.hpp -- gfx950 device building blocks of the MLP GEMM chain.
//
// One tile of either GEMM is computed by the same code in every kernel (the
// stream-ordered pair and the persistent kernel), so all policies produce
// bit-identical results:
//   * MFMA main loop: v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulators,
//     BK = 64 K-slab per step, K steps in ascending order, two LDS stages with
//     register prefetch of the next slab.
//   * LDS layout: every operand is stored K-contiguous, 8 chunks of 16 bytes
//     per row, with the chunk index XOR-swizzled by the row so that both the
//     16-byte fragment reads and the transposed writes avoid bank conflicts
//     (the bank-conflict motivation for swizzling is the jonahsamost bearblog
//     post on swizzling; the tile depth / staging discussion is its post on
//     adding depth to a GEMM).
//   * The weights are [K, N] row-major (N contiguous) while the matrix cores
//     want K-contiguous fragments, so each thread loads an 8x8 block of
//     16-bit values (eight 16-byte rows) and transposes it in registers with
//     byte permutes before the LDS store.
//   * Epilogue: activation on the fp32 accumulators, one round-to-nearest-even
//     conversion, staged through LDS and written with 16-byte stores (the
//     registers -> shared memory -> global (M, N) epilogue of the bearblog
//     post on epilogues).
//   * Tile synchronization (CuSync README, opening paragraph): producer tiles
//     publish per-tile ready flags with agent-scope release; consumer tiles
//     poll them with relaxed agent-scope loads and s_sleep back-off, then take
//     an agent-scope acquire fence before reading the intermediate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlpc {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { ACT_NONE = 0, ACT_GELU_TANH = 1, ACT_SWIGLU = 2 };
enum { DT_F16 = 0, DT_BF16 = 1 };
enum { POL_STREAM = 0, POL_ROW = 1, POL_TILE = 2 };

constexpr int BK = 64;          // K slab per main-loop step (8 chunks of 8 elements)
constexpr uint32_t NO_SKIP = 0xffffffffu;

// Kernel arguments shared by all kernels (passed by value).
struct ChainArgs {
    const uint16_t* x;      // [M, H]
    const uint16_t* w1;     // [H, g*I]
    const uint16_t* w2;     // [I, H]
    uint16_t* t;            // [M, I] intermediate (workspace)
    uint16_t* y;            // [M, H]
    int M, H, I;
    int act;
    uint32_t Mt, N1t, N2t, T1, T2;
    uint32_t group_m;       // row blocks per swizzle group
    uint32_t* ticket;       // tile queue counter
    uint32_t* flags;        // [Mt * N1t] ready epochs (tile_sync)
    uint32_t* rowcnt;       // [Mt] producer completions (row_sync)
    uint32_t* status;       // sticky watchdog status (nonzero = a consumer gave up)
    uint32_t ticket_base;   // tickets drawn by earlier runs (mod 2^32)
    uint32_t epoch;         // this run's epoch (mod 2^32)
    uint32_t grid;          // persistent workgroups
    uint32_t spin_limit;    // back-off iterations before a consumer gives up
    uint32_t skip_producer; // test hook: producer ticket that does nothing (NO_SKIP = none)
    int policy;
};

// Tile configuration.  BN is the output width of a tile; a SwiGLU producer
// tile holds 2*BN weight columns (gate and up) and two accumulator sets.
template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16x16");
    // bytes of one LDS stage for a B tile of gb*BN columns
    static constexpr int stage_bytes(int gb) { return (BM + gb * BN) * BK * 2; }
    static constexpr int lds_bytes(int gb) {
        int ml = 2 * stage_bytes(gb);
        int ep = BM * (BN + 8) * 2;
        return ml > ep ? ml : ep;
    }
};

// ------------------------------------------------------------------ helpers

// Byte offset of 16-byte chunk `c` (0..7) of LDS row `r` (rows of 64 elements).
__device__ __forceinline__ int lds_off(int r, int c) {
    return (r * 8 + (c ^ ((r ^ (r >> 3)) & 7))) * 16;
}

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DT == DT_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

// fp32 -> storage dtype, round to nearest even, from a value that has been
// rounded to fp32 first.  The empty asm pins `v` as an fp32 register value:
// without it the compiler may fuse the multiply that produced `v` with the
// conversion (v_fma_mixlo_f16), which rounds once instead of twice and makes
// the result depend on how the epilogue was inlined into each kernel.
template <int DT>
__device__ __forceinline__ uint16_t to_storage(float v) {
    asm volatile("" : "+v"(v));
    if constexpr (DT == DT_F16) {
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    } else {
        return __builtin_bit_cast(uint16_t, (__bf16)v);
    }
}

__device__ __forceinline__ float gelu_tanh(float h) {
    const float c = 0.7978845608028654f;   // sqrt(2/pi)
    const float k = 0.044715f;
    float inner = c * (h + k * (h * h * h));
    return 0.5f * h * (1.0f + tanhf(inner));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ u32x4 lds_ld16(const char* smem, int off) {
    return *reinterpret_cast<const u32x4*>(smem + off);
}

__device__ __forceinline__ void lds_st16(char* smem, int off, u32x4 v) {
    *reinterpret_cast<u32x4*>(smem + off) = v;
}

// Grouped tile order: walk GROUP row blocks down one column block before
// moving to the next column block, so tiles that run together share weight
// columns (and the activation rows) in L2 / MALL.
__device__ __forceinline__ void tile_coords(uint32_t t, uint32_t Mt, uint32_t Nt, uint32_t group,
                                            uint32_t& mb, uint32_t& nb) {
    const uint32_t per_group = group * Nt;
    const uint32_t gi = t / per_group;
    const uint32_t first = gi * group;
    const uint32_t gsz = (Mt - first) < group ? (Mt - first) : group;
    const uint32_t r = t - gi * per_group;
    mb = first + r % gsz;
    nb = r / gsz;
}

// ------------------------------------------------------------ flags / ticket

__device__ __forceinline__ uint32_t atomic_load_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-level wait: lane 0 polls `*p` until (int)(*p - target) >= 0, with
// s_sleep back-off, giving up after `limit` polls or when another consumer
// has already given up (status != 0).  Afterwards the whole wave takes an
// agent-scope acquire fence so its later loads see the producer's data.
// Returns true if the condition was met.
__device__ __forceinline__ bool wave_wait_geq(const uint32_t* p, uint32_t target, uint32_t* status,
                                              uint32_t limit) {
    const int lane = threadIdx.x & 63;
    uint32_t ok = 1;
    if (lane == 0) {
        uint32_t v = atomic_load_relaxed(p);
        if ((int32_t)(v - target) < 0) {
            uint32_t n = 0;
            for (;;) {
                __builtin_amdgcn_s_sleep(2);
                v = atomic_load_relaxed(p);
                if ((int32_t)(v - target) >= 0) break;
                if (++n >= limit || atomic_load_relaxed(status) != 0) {
                    __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = 0;
                    break;
                }
            }
        }
    }
    ok = __builtin_amdgcn_readfirstlane(ok);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return ok != 0;
}

// ---------------------------------------------------------------- main loop

// Loads of one BK slab into registers.
//  A: [rows, K] row-major, tile rows m0..m0+BM-1 (rows >= a_rows read as 0)
//  B: [K, ldb] row-major; tile column block n0..n0+BN-1 (and, for GB == 2, the
//     up block at column b_up + n0...), columns >= b_cols (per half) read as 0.
template <class C, int GB>
struct SlabRegs {
    static constexpr int A_CHUNKS = C::BM * 8;                          // 16-byte chunks
    static constexpr int A_IT = (A_CHUNKS + C::NT - 1) / C::NT;
    static constexpr int B_UNITS = 8 * (GB * C::BN / 8);                // 8x8 blocks
    static constexpr int B_IT = (B_UNITS + C::NT - 1) / C::NT;
    u32x4 a[A_IT];
    u32x4 b[B_IT][8];
};

template <class C, int GB>
__device__ __forceinline__ void load_a(SlabRegs<C, GB>& r, const uint16_t* A, int lda, int a_rows,
                                       int m0, int K, int k0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < SlabRegs<C, GB>::A_IT; ++i) {
        const int j = tid + i * C::NT;
        const int row = j >> 3, c = j & 7;
        const int gm = m0 + row, gk = k0 + c * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j < SlabRegs<C, GB>::A_CHUNKS && gm < a_rows && gk < K)
            v = ld16(A + (size_t)gm * lda + gk);
        r.a[i] = v;
    }
}

template <class C, int GB>
__device__ __forceinline__ void load_b(SlabRegs<C, GB>& r, const uint16_t* B, int ldb, int b_cols,
                                       int n0, int b_up, int K, int k0) {
    const int tid = threadIdx.x;
    constexpr int NB = GB * C::BN / 8;       // 8-column blocks across the (gate|up) tile
#pragma unroll
    for (int i = 0; i < SlabRegs<C, GB>::B_IT; ++i) {
        const int u = tid + i * C::NT;
        const int nb = u % NB, kb = u / NB;
        const int half = (GB == 2 && nb >= NB / 2) ? 1 : 0;
        const int nloc = (nb - half * (NB / 2)) * 8;          // column within the half
        const int gn = n0 + nloc;
        const int gcol = gn + half * b_up;
        const bool colok = (u < SlabRegs<C, GB>::B_UNITS) && gn < b_cols;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int gk = k0 + kb * 8 + rr;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (colok && gk < K) v = ld16(B + (size_t)gk * ldb + gcol);
            r.b[i][rr] = v;
        }
    }
}

template <class C, int GB>
__device__ __forceinline__ void store_slab(const SlabRegs<C, GB>& r, char* stage) {
    const int tid = threadIdx.x;
    char* sa = stage;
    char* sb = stage + C::BM * BK * 2;
#pragma unroll
    for (int i = 0; i < SlabRegs<C, GB>::A_IT; ++i) {
        const int j = tid + i * C::NT;
        if (j < SlabRegs<C, GB>::A_CHUNKS) lds_st16(sa, lds_off(j >> 3, j & 7), r.a[i]);
    }
    constexpr int NB = GB * C::BN / 8;
#pragma unroll
    for (int i = 0; i < SlabRegs<C, GB>::B_IT; ++i) {
        const int u = tid + i * C::NT;
        if (u < SlabRegs<C, GB>::B_UNITS) {
            const int nb = u % NB, kb = u / NB;
            // r.b[i][k] holds B[k][n0..n0+7] as 4 dwords, dword q = (col 2q | col 2q+1 << 16).
            // Output row n (= 2q + s) needs B[0..7][n] packed as dwords (k 2p | k 2p+1 << 16).
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4 lo, hi;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t e = r.b[i][2 * p][q];
                    const uint32_t o = r.b[i][2 * p + 1][q];
                    lo[p] = __builtin_amdgcn_perm(o, e, 0x05040100u);   // low halves
                    hi[p] = __builtin_amdgcn_perm(o, e, 0x07060302u);   // high halves
                }
                lds_st16(sb, lds_off(nb * 8 + 2 * q, kb), lo);
                lds_st16(sb, lds_off(nb * 8 + 2 * q + 1, kb), hi);
            }
        }
    }
}

template <class C, int DT, int GB>
__device__ __forceinline__ void compute_slab(const char* stage, f32x4 (&acc)[GB][C::FM][C::FN]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const char* sa = stage;
    const char* sb = stage + C::BM * BK * 2;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int chunk = kk * 4 + (lane >> 4);
        u32x4 af[C::FM];
        u32x4 bf[GB][C::FN];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
            af[fm] = lds_ld16(sa, lds_off(wm * C::WTM + fm * 16 + (lane & 15), chunk));
#pragma unroll
        for (int g = 0; g < GB; ++g)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
                bf[g][fn] = lds_ld16(sb, lds_off(g * C::BN + wn * C::WTN + fn * 16 + (lane & 15), chunk));
#pragma unroll
        for (int g = 0; g < GB; ++g)
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn)
                    acc[g][fm][fn] = mfma16x16x32<DT>(af[fm], bf[g][fn], acc[g][fm][fn]);
    }
}

// The K loop of one tile.  `wait(ks)` is called by every wave before the
// A-operand loads of slab ks (the consumer's dependency on the producer);
// the B-operand (weight) loads of that slab are issued before the wait.
template <class C, int DT, int GB, class Wait>
__device__ __forceinline__ void tile_mainloop(const uint16_t* A, int lda, int a_rows, int m0,
                                              const uint16_t* B, int ldb, int b_cols, int n0, int b_up,
                                              int K, f32x4 (&acc)[GB][C::FM][C::FN], char* smem,
                                              Wait&& wait) {
#pragma unroll
    for (int g = 0; g < GB; ++g)
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) acc[g][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int SB = C::stage_bytes(GB);
    const int nks = (K + BK - 1) / BK;
    SlabRegs<C, GB> r;
    load_b<C, GB>(r, B, ldb, b_cols, n0, b_up, K, 0);
    wait(0);
    load_a<C, GB>(r, A, lda, a_rows, m0, K, 0);
    store_slab<C, GB>(r, smem);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
        char* cur = smem + (ks & 1) * SB;
        char* nxt = smem + ((ks + 1) & 1) * SB;
        const bool more = ks + 1 < nks;
        if (more) {
            load_b<C, GB>(r, B, ldb, b_cols, n0, b_up, K, (ks + 1) * BK);
            wait(ks + 1);
            load_a<C, GB>(r, A, lda, a_rows, m0, K, (ks + 1) * BK);
        }
        compute_slab<C, DT, GB>(cur, acc);
        if (more) store_slab<C, GB>(r, nxt);
        __syncthreads();
    }
}

// Epilogue: activation on the fp32 accumulators, RNE to the storage dtype,
// staged through LDS, 16-byte stores of rows < rows and columns < cols.
template <class C, int DT, int GB>
__device__ __forceinline__ void tile_epilogue(const f32x4 (&acc)[GB][C::FM][C::FN], int act,
                                              uint16_t* D, int ldd, int rows, int cols, int m0, int n0,
                                              char* smem) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    constexpr int LD = C::BN + 8;     // padded LDS row (elements)
    uint16_t* s = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v;
                if constexpr (GB == 2) {
                    v = silu(acc[0][fm][fn][i]) * acc[1][fm][fn][i];
                } else {
                    v = acc[0][fm][fn][i];
                    if (act == ACT_GELU_TANH) v = gelu_tanh(v);
                }
                const int row = wm * C::WTM + fm * 16 + (lane >> 4) * 4 + i;
                const int col = wn * C::WTN + fn * 16 + (lane & 15);
                s[row * LD + col] = to_storage<DT>(v);
            }
    __syncthreads();
    constexpr int CHUNKS = C::BM * C::BN / 8;
    for (int j = threadIdx.x; j < CHUNKS; j += C::NT) {
        const int row = j / (C::BN / 8), c = j % (C::BN / 8);
        const int gm = m0 + row, gn = n0 + c * 8;
        if (gm < rows && gn < cols) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(s + row * LD + c * 8);
            st16(D + (size_t)gm * ldd + gn, v);
        }
    }
    __syncthreads();   // the staging area is free again for the next tile
}

struct NoWait {
    __device__ __forceinline__ void operator()(int) const {}
};

// Producer tile (GEMM1 + activation) writing T; returns after the stores.
template <class C, int DT, int GB>
__device__ __forceinline__ void producer_tile(const ChainArgs& a, uint32_t mb, uint32_t nb, char* smem) {
    f32x4 acc[GB][C::FM][C::FN];
    const int m0 = (int)mb * C::BM, n0 = (int)nb * C::BN;
    tile_mainloop<C, DT, GB>(a.x, a.H, a.M, m0, a.w1, GB * a.I, a.I, n0, a.I, a.H, acc, smem, NoWait{});
    tile_epilogue<C, DT, GB>(acc, a.act, a.t, a.I, a.M, a.I, m0, n0, smem);
}

// Consumer tile (GEMM2) reading T, writing Y.
template <class C, int DT, class Wait>
__device__ __forceinline__ void consumer_tile(const ChainArgs& a, uint32_t mb, uint32_t nb, char* smem,
                                              Wait&& wait) {
    f32x4 acc[1][C::FM][C::FN];
    const int m0 = (int)mb * C::BM, n0 = (int)nb * C::BN;
    tile_mainloop<C, DT, 1>(a.t, a.I, a.M, m0, a.w2, a.H, a.H, n0, 0, a.I, acc, smem, wait);
    tile_epilogue<C, DT, 1>(acc, ACT_NONE, a.y, a.H, a.M, a.H, m0, n0, smem);
}

}  // namespace mlpc
