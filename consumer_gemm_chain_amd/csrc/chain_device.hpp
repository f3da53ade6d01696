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

// Tile configuration: BM x BN tile, WM x WN waves of (BM/WM) x (BN/WN).  BN
// is the number of B (weight) columns of a tile: its output width, except
// for SwiGLU producer tiles, whose BN columns are gate/up pairs of BN/2
// output columns.
template <int BM_, int BN_, int WM_, int WN_, int OCC_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    // waves per SIMD the persistent kernel is register-limited to (the
    // occupancy of the standalone GEMM2 kernel of the same tile)
    static constexpr int OCC = OCC_;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16x16");
    static_assert(FN % 2 == 0, "SwiGLU tiles pair gate/up fragments within a wave");
    // bytes of one LDS stage (A tile and B tile of one BK slab)
    static constexpr int stage_bytes() { return (BM + BN) * BK * 2; }
    static constexpr int lds_bytes() {
        int ml = 2 * stage_bytes();
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

// Number of consecutive ready flags starting at index `from` (of `n`),
// polled by one whole wave: lane i reads flag from+i with a relaxed
// agent-scope load, and a ballot counts the leading run of flags that carry
// `epoch`.  Windows of 64 flags are scanned until one is not full.
__device__ __forceinline__ uint32_t wave_count_ready(const uint32_t* flags, uint32_t from, uint32_t n,
                                                     uint32_t epoch) {
    const uint32_t lane = threadIdx.x & 63;
    uint32_t r = from;
    while (r < n) {
        const uint32_t idx = r + lane;
        bool ok = false;
        if (idx < n) ok = (int32_t)(atomic_load_relaxed(flags + idx) - epoch) >= 0;
        const uint64_t b = __ballot(ok);
        const uint32_t lead = (~b == 0) ? 64u : (uint32_t)__builtin_ctzll(~b);
        r += lead;
        if (lead < 64) break;
    }
    return r < n ? r : n;
}

// Called by ONE whole wave: flags [0, from) are already acquired; wait
// until flags from..need are all ready (polling from `from`, s_sleep
// back-off), then take an agent-scope acquire fence so that the workgroup's
// later loads see the producers' data.  Returns the first flag index not
// known ready (> need), or n if the wait gave up (status records it).
__device__ __forceinline__ uint32_t wave_acquire_flags(const uint32_t* flags, uint32_t from, uint32_t need,
                                                       uint32_t n, uint32_t epoch, uint32_t* status,
                                                       uint32_t limit) {
    uint32_t r = wave_count_ready(flags, from, n, epoch);
    uint32_t polls = 0;
    while (r <= need) {
        __builtin_amdgcn_s_sleep(2);
        r = wave_count_ready(flags, r, n, epoch);
        if (r <= need && (++polls >= limit || atomic_load_relaxed(status) != 0)) {
            if ((threadIdx.x & 63) == 0)
                __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            r = n;
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return r;
}

// Called by ONE whole wave: wait until the counter reaches `target`
// ((int32)(count - target) >= 0), then acquire.  Returns false on timeout.
__device__ __forceinline__ bool wave_acquire_count(const uint32_t* cnt, uint32_t target, uint32_t* status,
                                                   uint32_t limit) {
    bool ok = true;
    uint32_t polls = 0;
    while ((int32_t)(atomic_load_relaxed(cnt) - target) < 0) {
        __builtin_amdgcn_s_sleep(2);
        if (++polls >= limit || atomic_load_relaxed(status) != 0) {
            if ((threadIdx.x & 63) == 0)
                __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = false;
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return ok;
}

// ---------------------------------------------------------------- main loop

// One tile's operands.  The same main loop serves both GEMMs, so producer
// and consumer tiles of the persistent kernel share one copy of the code.
//   A: [a_rows, K] row-major (lda), tile rows m0..m0+BM-1; rows >= a_rows read as 0
//   B: [K, ldb] row-major.  The tile's BN B-columns are, for a plain tile,
//      the output columns n0..n0+BN-1; for an interleaved (SwiGLU) tile the
//      16-column fragments alternate gate / up: fragment 2j is output
//      columns n0+16j..n0+16j+15 of the gate half, fragment 2j+1 the same
//      output columns of the up half (global column + up).  Output columns
//      >= b_cols read as 0.
struct TileJob {
    const uint16_t* A;
    const uint16_t* B;
    int lda, a_rows, m0;
    int ldb, b_cols, n0, up;
    int K;
    bool inter;
};

template <class C>
struct SlabRegs {
    static constexpr int A_CHUNKS = C::BM * 8;                          // 16-byte chunks
    static constexpr int A_IT = (A_CHUNKS + C::NT - 1) / C::NT;
    static constexpr int B_UNITS = C::BN;                              // 8x8 blocks: BN/8 columns x 8 k-rows
    static constexpr int B_IT = (B_UNITS + C::NT - 1) / C::NT;
    u32x4 a[A_IT];
    u32x4 b[B_IT][8];
};

// Global column of B-tile column block nb (8 columns) and whether it is in range.
__device__ __forceinline__ int b_column(const TileJob& j, int nb, bool& ok) {
    if (j.inter) {
        const int f = nb >> 1;                                   // 16-column fragment
        const int oc = j.n0 + (f >> 1) * 16 + (nb & 1) * 8;       // output column
        ok = oc < j.b_cols;
        return oc + (f & 1) * j.up;
    }
    const int oc = j.n0 + nb * 8;
    ok = oc < j.b_cols;
    return oc;
}

template <class C>
__device__ __forceinline__ void load_slab(SlabRegs<C>& r, const TileJob& j, int k0, bool do_a, bool do_b) {
    const int tid = threadIdx.x;
    if (do_b) {
        constexpr int NB = C::BN / 8;
#pragma unroll
        for (int i = 0; i < SlabRegs<C>::B_IT; ++i) {
            const int u = tid + i * C::NT;
            const int nb = u % NB, kb = u / NB;
            bool ok;
            const int gcol = b_column(j, nb, ok);
            ok = ok && (u < SlabRegs<C>::B_UNITS);
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int gk = k0 + kb * 8 + rr;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (ok && gk < j.K) v = ld16(j.B + (size_t)gk * j.ldb + gcol);
                r.b[i][rr] = v;
            }
        }
    }
    if (do_a) {
#pragma unroll
        for (int i = 0; i < SlabRegs<C>::A_IT; ++i) {
            const int q = tid + i * C::NT;
            const int row = q >> 3, c = q & 7;
            const int gm = j.m0 + row, gk = k0 + c * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (q < SlabRegs<C>::A_CHUNKS && gm < j.a_rows && gk < j.K)
                v = ld16(j.A + (size_t)gm * j.lda + gk);
            r.a[i] = v;
        }
    }
}

template <class C>
__device__ __forceinline__ void store_slab(const SlabRegs<C>& r, char* stage) {
    const int tid = threadIdx.x;
    char* sa = stage;
    char* sb = stage + C::BM * BK * 2;
#pragma unroll
    for (int i = 0; i < SlabRegs<C>::A_IT; ++i) {
        const int q = tid + i * C::NT;
        if (q < SlabRegs<C>::A_CHUNKS) lds_st16(sa, lds_off(q >> 3, q & 7), r.a[i]);
    }
    constexpr int NB = C::BN / 8;
#pragma unroll
    for (int i = 0; i < SlabRegs<C>::B_IT; ++i) {
        const int u = tid + i * C::NT;
        if (u < SlabRegs<C>::B_UNITS) {
            const int nb = u % NB, kb = u / NB;
            // r.b[i][k] holds B[k][8 columns] as 4 dwords, dword q = (col 2q | col 2q+1 << 16).
            // LDS row n (= 2q + s) needs B[0..7][n] packed as dwords (k 2p | k 2p+1 << 16).
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

template <class C, int DT>
__device__ __forceinline__ void compute_slab(const char* stage, f32x4 (&acc)[C::FM][C::FN]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const char* sa = stage;
    const char* sb = stage + C::BM * BK * 2;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int chunk = kk * 4 + (lane >> 4);
        u32x4 af[C::FM];
        u32x4 bf[C::FN];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
            af[fm] = lds_ld16(sa, lds_off(wm * C::WTM + fm * 16 + (lane & 15), chunk));
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
            bf[fn] = lds_ld16(sb, lds_off(wn * C::WTN + fn * 16 + (lane & 15), chunk));
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
                acc[fm][fn] = mfma16x16x32<DT>(af[fm], bf[fn], acc[fm][fn]);
    }
}

// The K loop of one tile.  `wait(ks)` is called (uniformly) before the
// A-operand loads of slab ks -- the consumer's dependency on its producers;
// the B-operand (weight) loads of that slab are issued before the wait.
template <class C, int DT, class Wait>
__device__ __forceinline__ void tile_mainloop(const TileJob& j, f32x4 (&acc)[C::FM][C::FN], char* smem,
                                              Wait&& wait) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int SB = C::stage_bytes();
    const int nks = (j.K + BK - 1) / BK;
    SlabRegs<C> r;
    load_slab<C>(r, j, 0, false, true);
    wait(0);
    load_slab<C>(r, j, 0, true, false);
    store_slab<C>(r, smem);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
        char* cur = smem + (ks & 1) * SB;
        char* nxt = smem + ((ks + 1) & 1) * SB;
        const bool more = ks + 1 < nks;
        if (more) {
            load_slab<C>(r, j, (ks + 1) * BK, false, true);
            wait(ks + 1);
            load_slab<C>(r, j, (ks + 1) * BK, true, false);
        }
        compute_slab<C, DT>(cur, acc);
        if (more) store_slab<C>(r, nxt);
        __syncthreads();
    }
}

// Epilogue: activation on the fp32 accumulators, RNE to the storage dtype,
// staged through LDS, 16-byte stores of rows < rows and columns < cols.
// For an interleaved (SwiGLU) tile, fragment pairs (2j, 2j+1) hold gate and
// up of the same output columns and the tile is BN/2 columns wide.
template <class C, int DT>
__device__ __forceinline__ void tile_epilogue(const f32x4 (&acc)[C::FM][C::FN], int act, bool inter,
                                              uint16_t* D, int ldd, int rows, int cols, int m0, int n0,
                                              char* smem) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    constexpr int LD = C::BN + 8;     // padded LDS row (elements)
    uint16_t* s = reinterpret_cast<uint16_t*>(smem);
    if (inter) {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; fn += 2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = silu(acc[fm][fn][i]) * acc[fm][fn + 1][i];
                    const int row = wm * C::WTM + fm * 16 + (lane >> 4) * 4 + i;
                    const int col = (wn * C::WTN + fn * 16) / 2 + (lane & 15);
                    s[row * LD + col] = to_storage<DT>(v);
                }
    } else {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = acc[fm][fn][i];
                    if (act == ACT_GELU_TANH) v = gelu_tanh(v);
                    const int row = wm * C::WTM + fm * 16 + (lane >> 4) * 4 + i;
                    const int col = wn * C::WTN + fn * 16 + (lane & 15);
                    s[row * LD + col] = to_storage<DT>(v);
                }
    }
    __syncthreads();
    const int width = inter ? C::BN / 2 : C::BN;
    const int cpr = width / 8;                    // 16-byte chunks per row
    for (int q = threadIdx.x; q < C::BM * cpr; q += C::NT) {
        const int row = q / cpr, c = q % cpr;
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

// Output width of a GEMM1 (producer) tile: BN, or BN/2 for SwiGLU.
template <class C>
__device__ __forceinline__ int producer_width(const ChainArgs& a) {
    return a.act == ACT_SWIGLU ? C::BN / 2 : C::BN;
}

template <class C>
__device__ __forceinline__ TileJob producer_job(const ChainArgs& a, uint32_t mb, uint32_t nb) {
    const bool inter = a.act == ACT_SWIGLU;
    return TileJob{a.x, a.w1, a.H, a.M, (int)mb * C::BM,
                   (inter ? 2 : 1) * a.I, a.I, (int)nb * producer_width<C>(a), inter ? a.I : 0,
                   a.H, inter};
}

template <class C>
__device__ __forceinline__ TileJob consumer_job(const ChainArgs& a, uint32_t mb, uint32_t nb) {
    return TileJob{a.t, a.w2, a.I, a.M, (int)mb * C::BM, a.H, a.H, (int)nb * C::BN, 0, a.I, false};
}

// One tile of either GEMM.  `role` 1 = producer (X W1 -> act -> T),
// 2 = consumer (T W2 -> Y); `wait` is only exercised by consumers.
template <class C, int DT, class Wait>
__device__ __forceinline__ void run_tile(const ChainArgs& a, int role, uint32_t mb, uint32_t nb, char* smem,
                                         Wait&& wait) {
    f32x4 acc[C::FM][C::FN];
    const TileJob j = role == 1 ? producer_job<C>(a, mb, nb) : consumer_job<C>(a, mb, nb);
    tile_mainloop<C, DT>(j, acc, smem, wait);
    if (role == 1)
        tile_epilogue<C, DT>(acc, a.act, j.inter, a.t, a.I, a.M, a.I, j.m0, j.n0, smem);
    else
        tile_epilogue<C, DT>(acc, ACT_NONE, false, a.y, a.H, a.M, a.H, j.m0, j.n0, smem);
}

}  // namespace mlpc
