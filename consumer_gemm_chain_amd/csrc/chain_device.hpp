// chain_device.hpp -- gfx950 device building blocks of the MLP GEMM chain.
//
// One tile of either GEMM is computed by the same code in every kernel (the
// stream-ordered pair and the persistent kernel), so all policies produce
// bit-identical results:
//   * MFMA main loop: v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulators,
//     BK = 64 K-slab per step, K steps in ascending order.
//   * Operand staging: both operands go from global memory straight into
//     LDS (global_load_lds_dwordx4, no registers) through a ring of NS LDS
//     stages, so up to NS-1 slabs are in flight while one is computed (the
//     pipeline depth of the jonahsamost bearblog post on adding depth to a
//     GEMM).  The ring is synchronized by explicit vmcnt waits and bare
//     barriers.  All main-loop LDS reads are inline asm with explicit
//     lgkmcnt waits: the compiler's wait-counter pass cannot tell an LDS
//     read of one stage from the DMA writes into another and would otherwise
//     wait for every DMA in flight (vmcnt(0)) before the first read of each
//     slab, draining the ring.
//   * Fragment double buffering: the MFMA fragments of the next half slab
//     are read from LDS while the MFMAs of the current half run.
//   * LDS layouts: the activation tile A is stored K-contiguous (8 chunks of
//     16 bytes per row) and read as MFMA fragments with ds_read_b128; the
//     weight tile B keeps the weights' [K, N] row-major layout and is read
//     with the gfx950 transpose read ds_read_b64_tr_b16 (each 16-lane group
//     reads a 4 x 16 block and receives it transposed).  Both use XOR chunk
//     swizzles, applied by choosing which global chunk each lane fetches,
//     against LDS bank conflicts (the bearblog post on swizzling).  The
//     swizzles depend only on the lane, so every fragment address is a
//     per-lane base plus a compile-time offset.
//   * Edges: rows past M and columns past N are clamped to the last valid
//     row / chunk (their results are never stored); a tile part whose K
//     range ends past K (only when K % 64 != 0) fetches out-of-range chunks
//     from a zero page, so the ring holds zeros beyond K.
//   * Epilogue: activation on the fp32 accumulators, one round-to-nearest-even
//     conversion, staged through LDS and written with 16-byte stores (the
//     registers -> shared memory -> global (M, N) epilogue of the bearblog
//     post on epilogues).
//   * Tile synchronization (CuSync README, opening paragraph): producer tiles
//     publish per-tile ready flags with agent-scope release; consumer tiles
//     poll them with relaxed agent-scope loads and s_sleep back-off, then take
//     the hand-off acquire (handoff_acquire: ordered loads, and an L2
//     invalidation only where producer tiles share 128-byte lines of the
//     intermediate) before reading it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
constexpr uint32_t MAX_LAYERS = 8;   // MLP layers of one chain (2 GEMMs each)

// Kernel arguments shared by all kernels (passed by value).
struct ChainArgs {
    const uint16_t* x;      // [M, H]
    const uint16_t* w1;     // [H, g*I]
    const uint16_t* w2;     // [I, H]
    uint16_t* t;            // [M, ldt] intermediate (workspace)
    uint16_t* y;            // [M, H]
    int M, H, I;
    int ldt;                // row stride of T: I rounded up to 64 elements (whole 128-byte lines per row)
    int act;
    uint32_t acq_agent;     // 1: producer tiles share 128-byte lines of T, hand-offs invalidate the L2
    uint32_t Mt, N1t, N2t, T1, T2;
    uint32_t rx;            // XCD grid rows (1, 2, 4 or 8; the grid is rx x 8/rx)
    uint32_t order;         // bit 0 / bit 1: GEMM1 / GEMM2 tiles walked column-major in each XCD block
    uint32_t* ticket;       // two sets of 8 tile-queue counters (one per XCD, 64 words apart), 512
                            // words apart: a fused run of epoch e uses set e & 1 (zero when it
                            // starts) and its workgroup 0 zeroes the other set
    uint64_t* run_epoch;    // fused runs: finished runs in the high 32 bits (the last finished run's
                            // epoch); the low half returns to its value at the end of each run
    uint32_t* flags;        // [8][fstride] ready epochs (tile_sync): one copy per XCD, each [Mt * N1t]
    uint32_t fstride;       // words between the XCDs' copies of the flags
    uint32_t* rowcnt;       // [Mt] producer completions (row_sync)
    uint32_t* status;       // sticky watchdog status (nonzero = a consumer gave up)
    const uint16_t* zero;   // >= 16 zero bytes: the source of every out-of-range chunk
    // deterministic split of each tile's K range (S1 parts per GEMM1 tile, S2
    // per GEMM2 tile; S = 1: no split).  Parts write fp32 partials; the last
    // part to arrive (per-tile counter, which it sets back to zero) sums them
    // in part order 0..S-1.
    uint32_t S1, S2;        // parts per tile
    uint32_t ksp1, ksp2;    // K slabs per part
    float* part1;           // [T1][S1][tile accumulators] (S1 > 1)
    float* part2;           // [T2][S2][tile accumulators] (S2 > 1)
    uint32_t* cnt1;         // [T1] part arrivals (S1 > 1), zero between executions
    uint32_t* cnt2;         // [T2] part arrivals (S2 > 1), zero between executions
    uint32_t* rdy1;         // [T1 * S1] part published (S1 > 1), zero between executions
    uint32_t* rdy2;         // [T2 * S2] part published (S2 > 1), zero between executions
    uint64_t* trace;        // optional timeline: 4 words per ticket (nullptr = off)
    uint32_t grid;          // persistent workgroups
    uint32_t spin_limit;    // back-off iterations before a consumer gives up
    uint32_t skip_producer; // test hook: producer ticket that does nothing (NO_SKIP = none)
    int policy;
    int ldx;                // row stride of x (GEMM1's A operand): H, or ldy for a later layer's input
    int ldo;                // row stride of y (GEMM2's output): H, or ldy for a layer's output kept for the next
    int ldw1, ldw2;         // row strides of every layer's W1 (>= g I) and W2 (>= H), in elements
    // Chains of several MLP layers (layers > 1): layer l computes
    // Y_l = act(Y_{l-1} W1_l) W2_l with Y_{-1} = x; the fields above then
    // describe layer 0, and layer_args() derives any layer's view.
    uint32_t layers;
    int ldy;                // row stride of the layer outputs kept in the workspace (H rounded up to 64)
    uint16_t* ys;           // [layers - 1][M, ldy]: Y_0 .. Y_{layers-2} (workspace)
    const uint16_t* w1s[MAX_LAYERS];
    const uint16_t* w2s[MAX_LAYERS];
};

// The arguments as layer l of a multi-layer chain sees them, for the
// stand-alone kernels of the stream-ordered policy (tile_elems: the fp32
// accumulators of one tile of the configuration): its weights, its input
// (x or the previous layer's output) and output (a kept layer output or y),
// its intermediate T_l, and its own split-K counters, ready words and
// partials -- the same buffers the multi-layer persistent kernel gives layer
// l (run_tile with l).  Layer 0 of a one-layer chain is the arguments
// themselves.
inline ChainArgs layer_args(const ChainArgs& a, uint32_t l, size_t tile_elems) {
    ChainArgs b = a;
    const size_t M = (size_t)a.M;
    if (l > 0) {
        b.x = a.ys + (l - 1) * M * (size_t)a.ldy;
        b.ldx = a.ldy;
    }
    if (l + 1 < a.layers) {
        b.y = a.ys + l * M * (size_t)a.ldy;
        b.ldo = a.ldy;
    }
    b.w1 = a.w1s[l];
    b.w2 = a.w2s[l];
    b.t = a.t + l * M * (size_t)a.ldt;
    b.cnt1 = a.cnt1 + l * a.T1;
    b.cnt2 = a.cnt2 + l * a.T2;
    b.rdy1 = a.rdy1 + l * a.T1 * a.S1;
    b.rdy2 = a.rdy2 + l * a.T2 * a.S2;
    if (a.part1) b.part1 = a.part1 + l * (size_t)a.T1 * a.S1 * tile_elems;
    if (a.part2) b.part2 = a.part2 + l * (size_t)a.T2 * a.S2 * tile_elems;
    // the stand-alone kernels see one layer whose buffers are the ones above
    b.layers = 1;
    return b;
}

// Tile configuration: BM x BN tile, WM x WN waves of (BM/WM) x (BN/WN), NS
// LDS stages of KS K-elements each (KS = 64: one slab per stage, read in two
// halves; KS = 32: half a slab per stage).  BN is the number of B (weight)
// columns of a tile: its output width, except for SwiGLU producer tiles,
// whose BN columns are gate/up pairs of BN/2 output columns.
template <int BM_, int BN_, int WM_, int WN_, int NS_, int OCC_, int KS_ = 64>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NS = NS_, KS = KS_;
    // waves per SIMD the persistent kernel is register-limited to
    static constexpr int OCC = OCC_;
    static constexpr int NW = WM * WN;
    static constexpr int NT = 64 * NW;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static_assert(KS == 64 || KS == 32, "K per stage: a slab or half a slab");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16x16");
    static_assert(FN % 2 == 0, "SwiGLU tiles pair gate/up fragments within a wave");
    static_assert(NS >= 2 && NS <= 14, "2 to 14 LDS stages");
    static_assert(KS == 64 || NS >= 3, "a ring of half slabs needs three stages");
    static_assert(KS == 64 || (BM * (KS / 8) / 64 / NW + KS * (BN / 8) / 64 / NW) * (NS - 1) <= 63,
                  "vmcnt range of a ring of half slabs");
    static constexpr int A_ROW = KS * 2;                 // bytes of one A row in a stage
    static constexpr int A_BYTES = BM * A_ROW;           // A stage: BM rows x KS elements
    static constexpr int B_BYTES = KS * BN * 2;          // B stage: KS k-rows x BN columns
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int RING = NS * STAGE;
    // epilogue staging (padded rows) in EPI_PASSES row passes that each fit the ring
    static constexpr int EPI_PASSES = BM * (BN + 8) * 2 <= RING ? 1 : BM * (BN + 8) * 2 <= 2 * RING ? 2 : 4;
    static constexpr int EPI_ROWS = BM / EPI_PASSES;
    static_assert(EPI_ROWS * (BN + 8) * 2 <= RING, "epilogue pass must fit the ring");
    static constexpr int CPR = BN / 8;                   // 16-byte chunks per B row
    static constexpr int A_PER_WAVE = BM * (KS / 8) / 64 / NW;   // 1 KB DMA instructions per wave per stage
    static constexpr int B_PER_WAVE = KS * CPR / 64 / NW;
    static_assert(A_PER_WAVE * NW * 64 == BM * (KS / 8) && B_PER_WAVE * NW * 64 == KS * CPR,
                  "DMA split across waves");
    static constexpr int LPS = A_PER_WAVE + B_PER_WAVE;  // DMA instructions per wave per stage
    static_assert(LPS * (NS - 2) <= 63, "vmcnt range");
    static constexpr int NREAD = FM + 2 * FN;            // LDS reads per fragment set
    // DMA of the next slab spread over the second half slab's MFMAs (eight
    // waves, at least three stages of a whole slab); otherwise issued in one
    // group after the first half slab's reads.  The spread form needs a
    // branch-free step, which made the compiler copy AGPR-resident
    // accumulators around the loop in the smaller configurations.
    static constexpr bool SPREAD = NW == 8 && NS >= 3 && KS == 64;
    static constexpr int lds_bytes() { return RING; }
};

// ------------------------------------------------------------------ helpers

// Test builds only (compiled with -DMLPC_CHAOS=1, a separate library that
// the tests load): a pseudo-random pause of up to about 16 us before a tile
// or a split part publishes, so that consumers and reducing parts meet
// their producers at shifted times.  Nothing in the normal build.
#ifndef MLPC_CHAOS
#define MLPC_CHAOS 0
#endif
__device__ __forceinline__ void chaos_delay(uint32_t key) {
#if MLPC_CHAOS
    uint32_t h = key * 0x9E3779B1u;
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    const uint32_t n = h & 63u;
    for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
#else
    (void)key;
#endif
}

// The thread's index in the workgroup, read afresh at each use: the empty
// volatile asm hands the compiler a new value each time, so nothing computed
// from it can be hoisted out of the persistent kernel's item loop.  (Hoisted,
// the per-lane DMA offsets, fragment addresses and epilogue indices of both
// tile roles stay live across every item and the 256 x 256 configuration
// spills them; recomputed per item they cost a few VALU instructions.)
__device__ __forceinline__ uint32_t thread_index() {
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// f(std::integral_constant<int, i>) for i = I .. N-1 (compile-time indices).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
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

// GeLU, tanh form: 0.5 h (1 + tanh u) with u = sqrt(2/pi) (h + 0.044715 h^3),
// evaluated as the identical h / (1 + exp(-2u)) through the hardware 2^x
// (v_exp_f32) and reciprocal (v_rcp_f32), about 1 ulp each -- a few fp32
// ulps in all, far below the rounding to the storage dtype that follows.
// Large negative u gives exp = inf and the result -0, as the tanh form does.
__device__ __forceinline__ float gelu_tanh(float h) {
    const float c = 0.7978845608028654f;   // sqrt(2/pi)
    const float k = 0.044715f;
    const float u = c * (h + k * (h * h * h));
    const float e = __builtin_amdgcn_exp2f(u * -2.8853900817779268f);   // exp(-2u) = 2^(-2u log2 e)
    return h * __builtin_amdgcn_rcpf(1.0f + e);
}

// SiLU g / (1 + exp(-g)), through the same hardware 2^x and reciprocal.
__device__ __forceinline__ float silu(float g) {
    const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);   // exp(-g)
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ u32x4 lds_ld16(const char* smem, int off) {
    return *reinterpret_cast<const u32x4*>(smem + off);
}


// Workgroups are dispatched to the 8 XCDs round-robin by index, and each XCD
// has its own L2.  Map index b to item (b % 8) * chunk + b / 8, so that each
// XCD gets one contiguous chunk of the item order (whose neighbouring tiles
// share weight panels and activation rows).  A bijection on [0, n).
__device__ __forceinline__ uint32_t xcd_chunked(uint32_t b, uint32_t n) {
    const uint32_t x = b & 7, i = b >> 3;
    const uint32_t q = n >> 3, r = n & 7;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// XCD partition of a GEMM's Mt x Nt tile grid (S parts per tile): the 8
// XCDs form an Rx x (8/Rx) grid and XCD x owns a contiguous block of row
// blocks and column blocks, walked with the parts of a tile adjacent, either
// row-major or column-major (CM).  Both GEMMs use the same row split, so the
// consumers of a row block sit on the XCDs whose producers complete it.  A
// block's weight panels and activation rows are shared in that XCD's L2 by
// the tiles that run there together: row-major finishes each row block
// early (for its consumers); column-major makes the ~32 tiles an XCD runs at
// once a (block rows) x (32 / block rows) patch, which shares more panels
// per K slab than one row of the block and a bit (for a 4 x 24 block of
// 256 x 128 tiles: 256 KB of distinct operands per slab instead of 448 KB).
struct XcdBlock {
    uint32_t r0, c0, nr, nc, len;    // first row block, first column block, rows, columns, items
};

__device__ __forceinline__ XcdBlock xcd_block(uint32_t Mt, uint32_t Nt, uint32_t S, uint32_t Rx, uint32_t x) {
    const uint32_t Cx = 8 / Rx;
    const uint32_t rx = x / Cx, cx = x % Cx;
    const uint32_t r0 = rx * Mt / Rx, r1 = (rx + 1) * Mt / Rx;
    const uint32_t c0 = cx * Nt / Cx, c1 = (cx + 1) * Nt / Cx;
    return XcdBlock{r0, c0, r1 - r0, c1 - c0, (r1 - r0) * (c1 - c0) * S};
}

// Item c of XCD block b -> tile (row block, column block) and part.
__device__ __forceinline__ void xcd_item(const XcdBlock& b, uint32_t S, bool cm, uint32_t c, uint32_t& mb,
                                         uint32_t& nb, uint32_t& part) {
    part = c % S;
    const uint32_t tc = c / S;
    if (cm) {
        mb = b.r0 + tc % b.nr;
        nb = b.c0 + tc / b.nr;
    } else {
        mb = b.r0 + tc / b.nc;
        nb = b.c0 + tc % b.nc;
    }
}

// Position p of the concatenation of the 8 XCD blocks -> tile and part.
__device__ __forceinline__ void xcd_position(uint32_t Mt, uint32_t Nt, uint32_t S, uint32_t Rx, bool cm, uint32_t p,
                                             uint32_t& mb, uint32_t& nb, uint32_t& part) {
    for (uint32_t x = 0; x < 8; ++x) {
        const XcdBlock b = xcd_block(Mt, Nt, S, Rx, x);
        if (p < b.len) {
            xcd_item(b, S, cm, p, mb, nb, part);
            return;
        }
        p -= b.len;
    }
    mb = nb = part = 0;   // not reached for p < Mt * Nt * S
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
    const uint32_t lane = thread_index() & 63;
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

// Acquire side of a producer -> consumer hand-off inside one launch.  The
// producer's release (agent scope) writes its data back to memory before it
// publishes the flag or count.  The consumer then only needs its own loads
// ordered after the flag load it observed, not an L2 invalidation, for a
// buffer that is written exactly once per launch, each 128-byte line of it
// by exactly one workgroup, and read only after that workgroup's release:
// the kernel dispatch invalidates the caches, so no line of such a buffer
// from an earlier launch can be cached, and no line of it is read before it
// is written.  The split-K partials always qualify (each part's region is a
// whole number of lines).  The intermediate T qualifies when each producer
// tile's columns cover whole lines: its row stride is a multiple of 64
// elements (the workspace pads it), so this holds when the producer tile is
// a multiple of 64 columns wide.  Narrower producer tiles (32 columns: the
// 16 x 64 configuration with SwiGLU) put two producers, possibly on two
// XCDs, in one line; an XCD whose L2 holds one producer's half of a line
// must not serve the other half from it, so those hand-offs (`agent`) take
// the agent-scope acquire (buffer_inv sc1: the XCD's L2 is invalidated).
// Elsewhere that invalidation would drop every other line of the XCD's L2
// -- the weight panels and activation rows the co-running tiles share --
// once per hand-off.
__device__ __forceinline__ void handoff_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup"); }

__device__ __forceinline__ void handoff_acquire(uint32_t agent) {
    if (agent) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Poll back-off: sleep `units` x 64 clocks, then double the interval up to
// POLL_MAX_UNITS (about 1 us).  Every consumer of a row block polls the
// same few flag lines with loads that bypass the L2; at a fixed short
// interval hundreds of waiting consumers concentrate enough traffic on
// those lines' memory channel to slow the producers they are waiting for.
constexpr uint32_t POLL_MAX_UNITS = 32;

__device__ __forceinline__ void poll_backoff(uint32_t& units) {
    for (uint32_t i = 0; i < units; ++i) __builtin_amdgcn_s_sleep(1);
    if (units < POLL_MAX_UNITS) units <<= 1;
}

// Called by ONE whole wave: flags [0, from) are already acquired; wait
// until flags from..need are all ready (polling from `from`, with
// back-off), then acquire (handoff_acquire) so that the workgroup's later
// loads see the producers' data.  Returns the first flag index not known
// ready (> need), or n if the wait gave up (status records it).
__device__ __forceinline__ uint32_t wave_acquire_flags(const uint32_t* flags, uint32_t from, uint32_t need,
                                                       uint32_t n, uint32_t epoch, uint32_t* status,
                                                       uint32_t limit, uint32_t agent) {
    uint32_t r = wave_count_ready(flags, from, n, epoch);
    uint32_t polls = 0, units = 1;
    while (r <= need) {
        poll_backoff(units);
        r = wave_count_ready(flags, r, n, epoch);
        if (r <= need && (++polls >= limit || atomic_load_relaxed(status) != 0)) {
            if ((thread_index() & 63) == 0)
                __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            r = n;
            break;
        }
    }
    handoff_acquire(agent);
    return r;
}

// Called by ONE whole wave: wait until the counter reaches `target`
// ((int32)(count - target) >= 0), then acquire.  Returns false on timeout.
__device__ __forceinline__ bool wave_acquire_count(const uint32_t* cnt, uint32_t target, uint32_t* status,
                                                   uint32_t limit, uint32_t agent) {
    bool ok = true;
    uint32_t polls = 0, units = 1;
    while ((int32_t)(atomic_load_relaxed(cnt) - target) < 0) {
        poll_backoff(units);
        if (++polls >= limit || atomic_load_relaxed(status) != 0) {
            if ((thread_index() & 63) == 0)
                __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = false;
            break;
        }
    }
    handoff_acquire(agent);
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
//   K slabs ks0..ks1-1 (BK = 64 each) are accumulated, in ascending order.
struct TileJob {
    const uint16_t* A;
    const uint16_t* B;
    const uint16_t* zero;
    int lda, a_rows, m0;
    int ldb, b_cols, n0, up;
    int K, ks0, ks1;
    bool inter;
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

// Global column of B-tile column block nb, with output columns past b_cols
// clamped to the last 8-column chunk (b_cols is a multiple of 8).
__device__ __forceinline__ int b_column_clamped(const TileJob& j, int nb) {
    if (j.inter) {
        const int f = nb >> 1;
        const int oc = min(j.n0 + (f >> 1) * 16 + (nb & 1) * 8, j.b_cols - 8);
        return oc + (f & 1) * j.up;
    }
    return min(j.n0 + nb * 8, j.b_cols - 8);
}

// The LDS ring of configuration C: NS stages of STAGE bytes (A slab, then B
// slab); stage 0 also holds the epilogue staging area.
template <class C>
__device__ __forceinline__ char* lds_ring() {
    __shared__ __attribute__((aligned(16))) char buf[C::lds_bytes()];
    return buf;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Physical 16-byte chunk of logical chunk c in A row r (8 chunks per row).
// A ds_read_b128 fragment read covers 16 consecutive rows (one chunk
// each).  XOR with r mod 8 reads free of LDS bank conflicts on gfx950
// (measured with the SQ_LDS_BANK_CONFLICT counter on this exact access
// pattern; variants that also mixed bit 3 of the row into the XOR
// conflicted two-way).  It depends on r mod 8 only, so fragments 16 rows
// apart are a fixed offset apart.
__device__ __forceinline__ int a_chunk(int r, int c) { return c ^ (r & 7); }

// The same for stages of half a slab (4 chunks of 16 bytes per A row): row r
// chunk c sits at physical chunk c ^ s(r), s(r) = r2 | (r1 ^ r3) << 1 (bit i
// of r is ri).  Any 16 consecutive rows then fill 16 distinct 16-byte slots
// of a 256-byte bank row, and any 8 of them starting at a multiple of 8 fill
// 8 distinct slots of a 128-byte one, so a ds_read_b128 fragment read (16
// rows, one chunk each) is free of bank conflicts whether the LDS serves
// 8 or 16 lanes per pass.  s depends on bits 1..3 of r only, so fragments
// 16 rows apart are a fixed offset apart.
__device__ __forceinline__ int a_chunk32(int r, int c) {
    return c ^ (((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1));
}

// Row and logical chunk of A-stage chunk position L (16-byte units) of
// configuration C: the global chunk a lane fetches into position L.
template <class C>
__device__ __forceinline__ void a_position(int L, int& r, int& c) {
    if constexpr (C::KS == 64) {
        r = L >> 3;
        c = a_chunk(r, L & 7);
    } else {
        r = L >> 2;
        c = a_chunk32(r, L & 3);
    }
}

// Physical chunk of logical chunk c in B row k.  A transpose read covers,
// per 32 lanes, rows 8g + (0..3) for g in {0,1} (or {2,3}) and two adjacent
// chunks per row; the XOR term 2*((k & 3) | ((k >> 3) & 1) << 2) gives those
// 8 rows 8 distinct chunk pairs, so the 32 lanes hit 64 distinct banks when
// a row has at least 16 chunks.
template <class C>
__device__ __forceinline__ int b_chunk(int k, int c) {
    return c ^ ((2 * ((k & 3) | (((k >> 3) & 1) << 2))) & (C::CPR - 1));
}

__device__ __forceinline__ void dma16(const void* src, char* lds) {
    // (a C-style cast is the way to change the address space to LDS)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}

// The wave index as a scalar (wave-uniform) value, so that LDS destinations
// built from it stay in scalar registers (M0 comes straight from them).
__device__ __forceinline__ int uniform_wave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A per-lane 32-bit offset re-materialised at its use: this keeps the
// compiler from hoisting its 64-bit extension out of the K loop, so that
// `uniform pointer + offset` selects the saddr form of the DMA (scalar base,
// 32-bit vector offset) instead of a 64-bit vector add per instruction.
__device__ __forceinline__ uint32_t fresh(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Per-tile DMA state of one lane.  A tile whose K range ends inside the
// matrices (every part except a last one with K % 64 != 0) is fetched in
// the saddr form of global_load_lds: a wave-uniform base pointer (scalar
// registers, advanced per slab) plus the lane's 32-bit byte offset of each
// chunk, computed once per tile, with no per-slab address arithmetic.  Rows
// past a_rows and columns past b_cols are clamped to the last row / column
// chunk: they read valid memory, and the results they produce are never
// stored.  A tile with a K tail takes the per-lane path with the zero page
// for every slab.
template <class C>
struct TileDma {
    const char* a_base;           // row m0 of A
    const char* b_base;           // B
    uint32_t va[C::A_PER_WAVE];   // A chunk offsets in slab 0 (bytes from a_base)
    uint32_t vb[C::B_PER_WAVE];   // B chunk offsets in slab 0 (bytes from b_base)
};

template <class C>
__device__ __forceinline__ TileDma<C> tile_dma(const TileJob& j) {
    TileDma<C> d;
    const int lane = thread_index() & 63, wave = thread_index() >> 6;
    d.a_base = reinterpret_cast<const char*>(j.A + (size_t)j.m0 * j.lda);
    d.b_base = reinterpret_cast<const char*>(j.B);
#pragma unroll
    for (int q = 0; q < C::A_PER_WAVE; ++q) {
        const int L = (wave * C::A_PER_WAVE + q) * 64 + lane;
        int r, c;
        a_position<C>(L, r, c);
        const int rr = min(j.m0 + r, j.a_rows - 1) - j.m0;
        d.va[q] = (uint32_t)rr * (uint32_t)j.lda * 2u + (uint32_t)c * 16u;
    }
#pragma unroll
    for (int q = 0; q < C::B_PER_WAVE; ++q) {
        const int L = (wave * C::B_PER_WAVE + q) * 64 + lane;
        const int k = L / C::CPR, p = L % C::CPR;
        const int gcol = b_column_clamped(j, b_chunk<C>(k, p));
        d.vb[q] = ((uint32_t)k * (uint32_t)j.ldb + (uint32_t)gcol) * 2u;
    }
    return d;
}

// Issue the DMA of K stage hs (K elements hs*KS .. hs*KS+KS-1; the slab
// itself when KS = 64) into ring stage `stage`, B part or A part.  Every
// wave issues B_PER_WAVE B instructions and A_PER_WAVE A instructions; lane
// i of an instruction fills LDS chunk L0 + i with the global chunk that
// belongs there under the swizzle.  TAIL: per-lane addresses, with the zero
// page for rows, columns and K indices outside the matrices.
template <class C, bool TAIL>
__device__ __forceinline__ void issue_b(const TileJob& j, const TileDma<C>& d, int hs, int stage) {
    char* st = lds_ring<C>() + stage * C::STAGE + C::A_BYTES;
    const int wave = uniform_wave();
    const int k0 = hs * C::KS;
    if constexpr (!TAIL) {
        const char* base = d.b_base + (size_t)k0 * j.ldb * 2;
#pragma unroll
        for (int q = 0; q < C::B_PER_WAVE; ++q)
            dma16(base + fresh(d.vb[q]), st + (wave * C::B_PER_WAVE + q) * 1024);
    } else {
        const int lane = thread_index() & 63;
#pragma unroll
        for (int q = 0; q < C::B_PER_WAVE; ++q) {
            const int L0 = (wave * C::B_PER_WAVE + q) * 64;
            const int L = L0 + lane;
            const int k = L / C::CPR, p = L % C::CPR;
            const int c = b_chunk<C>(k, p);
            bool ok;
            const int gcol = b_column(j, c, ok);
            const int gk = k0 + k;
            const uint16_t* src = (ok && gk < j.K) ? j.B + (size_t)gk * j.ldb + gcol : j.zero;
            dma16(src, st + L0 * 16);
        }
    }
}

template <class C, bool TAIL>
__device__ __forceinline__ void issue_a(const TileJob& j, const TileDma<C>& d, int hs, int stage) {
    char* st = lds_ring<C>() + stage * C::STAGE;
    const int wave = uniform_wave();
    const int k0 = hs * C::KS;
    if constexpr (!TAIL) {
        const char* base = d.a_base + (size_t)k0 * 2;
#pragma unroll
        for (int q = 0; q < C::A_PER_WAVE; ++q)
            dma16(base + fresh(d.va[q]), st + (wave * C::A_PER_WAVE + q) * 1024);
    } else {
        const int lane = thread_index() & 63;
#pragma unroll
        for (int q = 0; q < C::A_PER_WAVE; ++q) {
            const int L0 = (wave * C::A_PER_WAVE + q) * 64;
            const int L = L0 + lane;
            int r, c;
            a_position<C>(L, r, c);
            const int gm = j.m0 + r, gk = k0 + c * 8;
            const uint16_t* src = (gm < j.a_rows && gk < j.K) ? j.A + (size_t)gm * j.lda + gk : j.zero;
            dma16(src, st + L0 * 16);
        }
    }
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS fragment reads as inline asm: the result must not be used before
// lgkm_wait() and pin() (the MFMAs depend on the pinned values).
template <uint32_t OFF>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
    static_assert(OFF < 65536, "ds offset field");
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}

template <uint32_t OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_b64(uint32_t addr) {
    static_assert(OFF < 65536, "ds offset field");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}

// Wait until at most N LDS instructions of this wave are outstanding.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
    asm volatile("s_waitcnt lgkmcnt(%0)" :: "i"(N < 15 ? N : 15) : "memory");
}

template <class T>
__device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }

// One wave's MFMA operands for a 32-deep half slab.
template <class C>
struct Frags {
    u32x4 a[C::FM];
    u32x4 b[C::FN];
};

// Per-lane LDS byte addresses of the first fragments in stage 0: A
// fragment fm = 0 for each half slab kk, B fragment fn (half slab 0, rows
// k..k+3).  Every other fragment address is one of these plus a
// compile-time offset (stage, fm, kk, upper four rows).
template <class C>
struct FragBase {
    uint32_t a[2];
    uint32_t b[C::FN];
};

template <class C>
__device__ __forceinline__ FragBase<C> frag_base() {
    FragBase<C> f;
    const uint32_t ring = lds_addr(lds_ring<C>());
    const int lane = thread_index() & 63, wave = thread_index() >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int g = lane >> 4, jj = lane & 15;
    const int r = wm * C::WTM + jj;
    if constexpr (C::KS == 64) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) f.a[kk] = ring + (r * 8 + a_chunk(r, kk * 4 + g)) * 16;
    } else {
        f.a[0] = f.a[1] = ring + (r * 4 + a_chunk32(r, g)) * 16;
    }
    // lane (g, jj) of a transpose read: row k = 8g + jj/4 (+4 for the upper
    // rows, +32 for half slab 1 of a whole-slab stage), columns (jj%4)*4..+3
    // of the fragment.
    // b_chunk depends on k & 3 and (k >> 3) & 1 only, which neither +4 nor
    // +32 changes.
    const int k = g * 8 + (jj >> 2);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
        const int col = wn * C::WTN + fn * 16 + (jj & 3) * 4;
        const int c = col >> 3, half = (col & 7) * 2;
        f.b[fn] = ring + C::A_BYTES + (k * C::CPR + b_chunk<C>(k, c)) * 16 + half;
    }
    return f;
}

// Issue the LDS reads of half slab KK of the stage at byte offset `so` into f
// (KK = 0 for a stage of half a slab).
template <class C, int KK>
__device__ __forceinline__ void frag_load(const FragBase<C>& fb, uint32_t so, Frags<C>& f) {
    static_assert(KK == 0 || C::KS == 64, "a stage of half a slab has one half");
    constexpr uint32_t A_MAX = (C::FM - 1) * 16 * C::A_ROW;
    constexpr uint32_t B_MAX = (KK * 32 + 4) * C::CPR * 16;
    static_assert(A_MAX < 65536 && C::A_BYTES + B_MAX < 65536, "stage too large for ds offsets");
    const uint32_t a = fb.a[KK] + so;
    static_for<0, C::FM>([&](auto fm) { f.a[fm] = ds_read_b128<decltype(fm)::value * 16 * C::A_ROW>(a); });
    static_for<0, C::FN>([&](auto fn) {
        const uint32_t b = fb.b[fn] + so;
        const u32x2 lo = ds_read_tr16_b64<KK * 32 * C::CPR * 16>(b);
        const u32x2 hi = ds_read_tr16_b64<(KK * 32 + 4) * C::CPR * 16>(b);
        f.b[fn] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    });
}

// Make the fragment registers available to the MFMAs (after lgkm_wait).
template <class C>
__device__ __forceinline__ void frag_pin(Frags<C>& f) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) pin(f.a[fm]);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) pin(f.b[fn]);
}

template <class C, int DT>
__device__ __forceinline__ void mfma_block(f32x4 (&acc)[C::FM][C::FN], const Frags<C>& f) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = mfma16x16x32<DT>(f.a[fm], f.b[fn], acc[fm][fn]);
}

// Read number R (A fragments first, then the two halves of each B
// fragment) of half slab KK of the stage at byte offset `so` into f.
template <class C, int KK, int R>
__device__ __forceinline__ void frag_read_one(const FragBase<C>& fb, uint32_t so, Frags<C>& f) {
    if constexpr (R < C::FM) {
        f.a[R] = ds_read_b128<R * 16 * C::A_ROW>(fb.a[KK] + so);
    } else {
        constexpr int fn = (R - C::FM) / 2, hi = (R - C::FM) % 2;
        const u32x2 v = ds_read_tr16_b64<(KK * 32 + 4 * hi) * C::CPR * 16>(fb.b[fn] + so);
        if constexpr (hi == 0) {
            f.b[fn][0] = v[0];
            f.b[fn][1] = v[1];
        } else {
            f.b[fn][2] = v[0];
            f.b[fn][3] = v[1];
        }
    }
}

// Order of the NREAD reads of the second half slab (frag_read_one numbering:
// R < FM is A fragment R, the rest the B halves) among the first half's
// MFMAs (row fm = MFMAs fm*FN .. fm*FN+FN-1): A fragment fm right after the
// last MFMA of row fm -- the moment the first half's A fragment fm dies, so
// the compiler can give the new one the same registers -- and the B halves
// in the other slots, in order; B halves with no slot follow the block.
template <class C>
struct ReadPlan {
    int after[C::FM * C::FN];   // read issued after MFMA I, or -1
    int tail[C::NREAD];         // reads issued after the block
    int ntail;
    int pos[C::NREAD];          // issue position of each read
};

template <class C>
constexpr ReadPlan<C> read_plan() {
    ReadPlan<C> p{};
    int nb = 0, n = 0;
    for (int i = 0; i < C::FM * C::FN; ++i) {
        int r = -1;
        if (i % C::FN == C::FN - 1) r = i / C::FN;
        else if (nb < 2 * C::FN) r = C::FM + nb++;
        p.after[i] = r;
        if (r >= 0) p.pos[r] = n++;
    }
    p.ntail = 0;
    while (nb < 2 * C::FN) {
        p.tail[p.ntail++] = C::FM + nb;
        p.pos[C::FM + nb++] = n++;
    }
    return p;
}

// Reads of the second half slab still allowed in flight when row fm of its
// MFMAs starts (it needs A fragment fm and every B half).
template <class C>
constexpr int rows_wait(int fm) {
    constexpr ReadPlan<C> p = read_plan<C>();
    int last = p.pos[fm];
    for (int b = 0; b < 2 * C::FN; ++b)
        if (p.pos[C::FM + b] > last) last = p.pos[C::FM + b];
    return C::NREAD - 1 - last;
}

// The MFMAs of fragments f, with the reads of half slab KK into g issued
// among them in read_plan order.
template <class C, int DT, int KK>
__device__ __forceinline__ void mfma_block_reading(f32x4 (&acc)[C::FM][C::FN], const Frags<C>& f,
                                                   const FragBase<C>& fb, uint32_t so, Frags<C>& g) {
    constexpr ReadPlan<C> plan = read_plan<C>();
    static_for<0, C::FM * C::FN>([&](auto i) {
        constexpr int I = decltype(i)::value;
        acc[I / C::FN][I % C::FN] = mfma16x16x32<DT>(f.a[I / C::FN], f.b[I % C::FN], acc[I / C::FN][I % C::FN]);
        if constexpr (plan.after[I] >= 0) frag_read_one<C, KK, plan.after[I]>(fb, so, g);
        __builtin_amdgcn_sched_barrier(0);
    });
    static_for<0, plan.ntail>([&](auto t) { frag_read_one<C, KK, plan.tail[decltype(t)::value]>(fb, so, g); });
}

// Before the first MFMA of row fm of fragments g (read by
// mfma_block_reading): wait for what that row needs and make it available.
template <class C, int FMROW>
__device__ __forceinline__ void rows_ready(Frags<C>& g) {
    lgkm_wait<rows_wait<C>(FMROW)>();
    pin(g.a[FMROW]);
    if constexpr (FMROW == 0) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) pin(g.b[fn]);
    }
}

// The MFMAs of fragments g as they arrive (row by row).
template <class C, int DT>
__device__ __forceinline__ void mfma_block_rows(f32x4 (&acc)[C::FM][C::FN], Frags<C>& g) {
    static_for<0, C::FM * C::FN>([&](auto i) {
        constexpr int I = decltype(i)::value;
        if constexpr (I % C::FN == 0) rows_ready<C, I / C::FN>(g);
        acc[I / C::FN][I % C::FN] = mfma16x16x32<DT>(g.a[I / C::FN], g.b[I % C::FN], acc[I / C::FN][I % C::FN]);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Wait until at most `n` DMA instructions of this wave are outstanding and
// every LDS access of this wave has completed, then meet the other waves.
// (A bare s_barrier: __syncthreads() would also wait for all DMA.)
// The empty asm statements with a memory clobber and the scheduling
// barriers keep the compiler from moving any memory access across the
// barrier.
template <int N>
__device__ __forceinline__ void ring_barrier() {
    static_assert(N >= 0 && N <= 63, "vmcnt");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// LDS-visible barrier that leaves the DMA ring in flight.
__device__ __forceinline__ void lds_barrier() { ring_barrier<63>(); }

// DMA instruction Q (of LPS) of slab ks into stage `stage`: Q < B_PER_WAVE
// is B instruction Q, the rest are the A instructions.
template <class C, bool TAIL, int Q>
__device__ __forceinline__ void issue_one(const TileJob& j, const TileDma<C>& d, int hs, int stage) {
    const int wave = uniform_wave();
    const int k0 = hs * C::KS;
    if constexpr (Q < C::B_PER_WAVE) {
        char* st = lds_ring<C>() + stage * C::STAGE + C::A_BYTES;
        if constexpr (!TAIL) {
            const char* base = d.b_base + (size_t)k0 * j.ldb * 2;
            dma16(base + fresh(d.vb[Q]), st + (wave * C::B_PER_WAVE + Q) * 1024);
        } else {
            const int L0 = (wave * C::B_PER_WAVE + Q) * 64;
            const int L = L0 + (thread_index() & 63);
            const int k = L / C::CPR, p = L % C::CPR;
            bool ok;
            const int gcol = b_column(j, b_chunk<C>(k, p), ok);
            const int gk = k0 + k;
            dma16((ok && gk < j.K) ? j.B + (size_t)gk * j.ldb + gcol : j.zero, st + L0 * 16);
        }
    } else {
        constexpr int QA = Q - C::B_PER_WAVE;
        char* st = lds_ring<C>() + stage * C::STAGE;
        if constexpr (!TAIL) {
            const char* base = d.a_base + (size_t)k0 * 2;
            dma16(base + fresh(d.va[QA]), st + (wave * C::A_PER_WAVE + QA) * 1024);
        } else {
            const int L0 = (wave * C::A_PER_WAVE + QA) * 64;
            const int L = L0 + (thread_index() & 63);
            int r, c;
            a_position<C>(L, r, c);
            const int gm = j.m0 + r, gk = k0 + c * 8;
            dma16((gm < j.a_rows && gk < j.K) ? j.A + (size_t)gm * j.lda + gk : j.zero, st + L0 * 16);
        }
    }
}

// The MFMAs of fragments f with the LPS DMA instructions of slab ks (into
// `stage`) issued one after every other MFMA, so that the DMA of all waves
// is spread over the step instead of queueing up in one burst.
template <class C, int DT, bool TAIL>
__device__ __forceinline__ void mfma_block_dma(f32x4 (&acc)[C::FM][C::FN], Frags<C>& f,
                                               const TileJob& j, const TileDma<C>& d, int ks, int stage) {
    constexpr int GAP = (C::FM * C::FN) / C::LPS >= 2 ? 2 : 1;
    static_for<0, C::FM * C::FN>([&](auto i) {
        constexpr int I = decltype(i)::value;
        if constexpr (I % C::FN == 0) rows_ready<C, I / C::FN>(f);
        acc[I / C::FN][I % C::FN] = mfma16x16x32<DT>(f.a[I / C::FN], f.b[I % C::FN], acc[I / C::FN][I % C::FN]);
        if constexpr (I % GAP == 0 && I / GAP < C::LPS) issue_one<C, TAIL, I / GAP>(j, d, ks, stage);
        __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr ((C::FM * C::FN + GAP - 1) / GAP < C::LPS) {
        static_for<(C::FM * C::FN + GAP - 1) / GAP, C::LPS>([&](auto q) {
            issue_one<C, TAIL, decltype(q)::value>(j, d, ks, stage);
        });
    }
}

template <class C, bool TAIL, class Wait>
__device__ __forceinline__ void issue_slab(const TileJob& j, const TileDma<C>& d, int ks, int stage, Wait& wait) {
    issue_b<C, TAIL>(j, d, ks, stage);
    wait(ks);
    issue_a<C, TAIL>(j, d, ks, stage);
}

// The K loop of one tile over slabs ks0 .. ks1-1.  `wait(ks)` is called
// (uniformly) before the A-operand DMA of slab ks -- the consumer's
// dependency on its producers.  Slab ks0 + i lives in stage i % NS; slabs
// ks0 .. ks0+NS-2 are requested before the first step.  One step per slab
// ks (stage st):
//   barrier: slab ks has landed and every wave is done with the stage of
//     slab ks-1, which now takes slab ks+NS-1;
//   issue the reads of the first half slab (f0);
//   [not SPREAD: issue the DMA of slab ks+NS-1 -- it overlaps the reads]
//   wait for f0, then its MFMAs, with one read of the second half slab (f1)
//   issued after each of the first NREAD of them;
//   wait for f1, then its MFMAs [SPREAD: with the LPS DMA instructions of
//   slab ks+NS-1 issued after every other one].
// Issuing every wave's DMA in one group right after the barrier stalled the
// waves on the full memory queue for a large part of the step (measured with
// s_memtime around each phase); spread over the MFMAs the queue drains while
// the matrix cores work.  In the SPREAD form the step has no branch between
// the MFMAs: past the part's end the last slab is fetched again (into a stage
// that is never read), so the DMA count and the waits stay fixed; the other
// form skips those slabs and waits for every outstanding one instead.  (With
// the next slab's first half read during the second half's MFMAs and the
// barrier between the two MFMA groups, a step took 4-10% more cycles.)
template <class C, int DT, bool TAIL, class Wait>
__device__ __forceinline__ void tile_kloop(const TileJob& j, f32x4 (&acc)[C::FM][C::FN], Wait& wait) {
    const FragBase<C> fb = frag_base<C>();
    const TileDma<C> d = tile_dma<C>(j);
    const int ks0 = j.ks0, ks1 = j.ks1;
#pragma unroll
    for (int i = 0; i < C::NS - 1; ++i) {
        if constexpr (!C::SPREAD) {
            if (ks0 + i < ks1) issue_slab<C, TAIL, Wait>(j, d, ks0 + i, i, wait);
        } else {
            if (ks0 + i < ks1) wait(ks0 + i);
            const int kd = ks0 + i < ks1 ? ks0 + i : ks1 - 1;
            static_for<0, C::LPS>([&](auto q) { issue_one<C, TAIL, decltype(q)::value>(j, d, kd, i); });
        }
    }
    int st = 0;
    for (int ks = ks0; ks < ks1; ++ks) {
        const int pv = st == 0 ? C::NS - 1 : st - 1;
        const int kn = ks + C::NS - 1;
        Frags<C> f0, f1;
        if constexpr (!C::SPREAD) {
            // request slab ks+NS-1 right after this slab's first fragment
            // reads, once it is known to exist
            if (kn <= ks1) ring_barrier<C::LPS * (C::NS - 2)>();
            else ring_barrier<0>();
            frag_load<C, 0>(fb, (uint32_t)st * C::STAGE, f0);
            __builtin_amdgcn_sched_barrier(0);
            if (kn < ks1) issue_slab<C, TAIL, Wait>(j, d, kn, pv, wait);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            // slab ks+NS-1 goes into the stage of slab ks-1, its DMA spread
            // over the second half slab's MFMAs; past the part's end the
            // last slab is fetched again (never read), which keeps the DMA
            // count per step and the waits fixed and the MFMA groups free of
            // branches
            if (kn < ks1) wait(kn);
            ring_barrier<C::LPS * (C::NS - 2)>();
            frag_load<C, 0>(fb, (uint32_t)st * C::STAGE, f0);
            __builtin_amdgcn_sched_barrier(0);
        }
        lgkm_wait<0>();
        frag_pin(f0);
        mfma_block_reading<C, DT, 1>(acc, f0, fb, (uint32_t)st * C::STAGE, f1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!C::SPREAD) mfma_block_rows<C, DT>(acc, f1);
        else mfma_block_dma<C, DT, TAIL>(acc, f1, j, d, kn < ks1 ? kn : ks1 - 1, pv);
        __builtin_amdgcn_sched_barrier(0);
        st = st + 1 == C::NS ? 0 : st + 1;
    }
}

// The MFMAs of fragments f (a ring of half slabs), with the reads of the
// next stage's fragments into g issued among them in read_plan order and
// the LPS DMA instructions of K stage hr (into ring stage `stage`) issued
// after every other MFMA: weights first, then the consumer's wait for the
// slab (where the stage starts one), then the activations.
template <class C, int DT, bool TAIL, class Wait>
__device__ __forceinline__ void mfma_block_fine(f32x4 (&acc)[C::FM][C::FN], const Frags<C>& f, const FragBase<C>& fb,
                                                uint32_t so, Frags<C>& g, const TileJob& j, const TileDma<C>& d,
                                                int hr, int stage, Wait& wait) {
    constexpr ReadPlan<C> plan = read_plan<C>();
    constexpr int GAP = (C::FM * C::FN) / C::LPS >= 2 ? 2 : 1;
    constexpr int HPS = BK / C::KS;
    static_for<0, C::FM * C::FN>([&](auto i) {
        constexpr int I = decltype(i)::value;
        acc[I / C::FN][I % C::FN] = mfma16x16x32<DT>(f.a[I / C::FN], f.b[I % C::FN], acc[I / C::FN][I % C::FN]);
        if constexpr (plan.after[I] >= 0) frag_read_one<C, 0, plan.after[I]>(fb, so, g);
        if constexpr (I % GAP == 0 && I / GAP < C::LPS) {
            constexpr int Q = I / GAP;
            if constexpr (Q == C::B_PER_WAVE) {
                if (hr % HPS == 0) wait(hr / HPS);
            }
            issue_one<C, TAIL, Q>(j, d, hr, stage);
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    static_for<0, plan.ntail>([&](auto t) { frag_read_one<C, 0, plan.tail[decltype(t)::value]>(fb, so, g); });
    if constexpr ((C::FM * C::FN + GAP - 1) / GAP < C::LPS) {
        static_for<(C::FM * C::FN + GAP - 1) / GAP, C::LPS>([&](auto q) {
            constexpr int Q = decltype(q)::value;
            if constexpr (Q == C::B_PER_WAVE) {
                if (hr % HPS == 0) wait(hr / HPS);
            }
            issue_one<C, TAIL, Q>(j, d, hr, stage);
        });
    }
}

// The K loop over a ring of NS stages of half a slab (KS = 32).  K stage h
// (of 32 elements; a part's slabs ks0 .. ks1-1 are stages 2 ks0 .. 2 ks1 - 1)
// lives in ring stage (h - 2 ks0) % NS.  Stages h0 .. h0+NS-1 fill the ring
// before the first step and the fragments of stage h0 are read.  One step per
// stage h, its fragments in registers (f):
//   wait for this wave's reads of stage h, then for the DMA of stage h+1 in
//   every wave (barrier): the ring stage of h is free again;
//   the MFMAs of f, with the reads of stage h+1's fragments (g) and the DMA
//   of stage h+NS into the ring stage of h (weights first, then the
//   consumer's wait for the slab, then the activations) issued among them.
// So NS-1 stages are in flight while one is multiplied and the next one is
// read (three for NS = 4: 96 KB for 256 x 256 tiles, where a ring of two
// whole slabs has one slab, 64 KB), and no MFMA waits for its fragments
// after a barrier.  The number of steps is even, so the loop takes two per
// iteration and f and g swap roles without copies.
template <class C, int DT, bool TAIL, class Wait>
__device__ __forceinline__ void tile_kloop_fine(const TileJob& j, f32x4 (&acc)[C::FM][C::FN], Wait& wait) {
    static_assert(C::KS == 32 && C::NS >= 3, "ring of half slabs");
    constexpr int HPS = BK / C::KS;       // stages per slab
    const FragBase<C> fb = frag_base<C>();
    const TileDma<C> d = tile_dma<C>(j);
    const int h0 = j.ks0 * HPS, h1 = j.ks1 * HPS;
    auto request = [&](int h, int stage) {
        issue_b<C, TAIL>(j, d, h, stage);
        if (h % HPS == 0) wait(h / HPS);
        issue_a<C, TAIL>(j, d, h, stage);
    };
    // (a part shorter than the ring requests its last stage again into the
    // ring stages it does not use, so that every wave has issued the same
    // number of DMA instructions at every barrier)
#pragma unroll
    for (int i = 0; i < C::NS; ++i) request(h0 + i < h1 ? h0 + i : h1 - 1, i);
    Frags<C> f, g;
    // stage h0 landed in every wave
    ring_barrier<C::LPS * (C::NS - 1)>();
    frag_load<C, 0>(fb, 0u, f);
    __builtin_amdgcn_sched_barrier(0);
    int st = 0;
    auto step = [&](int h, Frags<C>& cur, Frags<C>& nxt) {
        const int sn = st + 1 == C::NS ? 0 : st + 1;
        lgkm_wait<0>();
        frag_pin(cur);
        // Every step requests one stage into the ring stage of h, so the
        // DMA count per step and the waits stay fixed: past the part's end
        // that is the part's last stage again (never read from there).
        ring_barrier<C::LPS * (C::NS - 2)>();
        const int hr = h + C::NS < h1 ? h + C::NS : h1 - 1;
        mfma_block_fine<C, DT, TAIL>(acc, cur, fb, (uint32_t)sn * C::STAGE, nxt, j, d, hr, st, wait);
        __builtin_amdgcn_sched_barrier(0);
        st = sn;
    };
    for (int h = h0; h < h1; h += 2) {
        step(h, f, g);
        step(h + 1, g, f);
    }
    // the last step's reads (never used) land before their registers can be
    // given to anything else
    lgkm_wait<0>();
    frag_pin(f);
}

template <class C, int DT, class Wait>
__device__ __forceinline__ void tile_mainloop(const TileJob& j, f32x4 (&acc)[C::FM][C::FN], Wait& wait) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j.ks1 > j.ks0) {
        if constexpr (C::KS == 32) {
            if (j.ks1 * BK <= j.K) tile_kloop_fine<C, DT, false>(j, acc, wait);
            else tile_kloop_fine<C, DT, true>(j, acc, wait);
        } else {
            if (j.ks1 * BK <= j.K) tile_kloop<C, DT, false>(j, acc, wait);
            else tile_kloop<C, DT, true>(j, acc, wait);
        }
    }
    // every wave is done reading the ring (and all DMA has landed) before
    // the epilogue reuses stage 0
    ring_barrier<0>();
}

// Epilogue: activation on the fp32 accumulators, RNE to the storage dtype,
// staged through LDS (stage 0, in EPI_PASSES passes of EPI_ROWS rows), and
// 16-byte stores of rows < rows and columns < cols.  For an interleaved
// (SwiGLU) tile, fragment pairs (2j, 2j+1) hold gate and up of the same
// output columns and the tile is BN/2 columns wide.
template <class C, int DT>
__device__ __forceinline__ void tile_epilogue(const f32x4 (&acc)[C::FM][C::FN], int act, bool inter,
                                              uint16_t* D, int ldd, int rows, int cols, int m0, int n0) {
    char* smem = lds_ring<C>();
    const int lane = thread_index() & 63;
    const int wave = thread_index() >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    constexpr int LD = C::BN + 8;     // padded LDS row (elements)
    uint16_t* s = reinterpret_cast<uint16_t*>(smem);
    const int width = inter ? C::BN / 2 : C::BN;
    const int cpr = width / 8;                    // 16-byte chunks per row
    // Activation and rounding of every fragment first, in every wave (the
    // staging passes below only cover some waves' rows each), kept as packed
    // 16-bit pairs: element i of fragment f in half i / 2 of pk[f][i / 2].
    constexpr int NV = C::FN;                     // value fragments per row (halved for SwiGLU)
    uint32_t pk[C::FM][NV][2];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < NV; ++fn)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t lo = 0, hi = 0;
                if (inter) {
                    if (fn < NV / 2) {
                        lo = to_storage<DT>(silu(acc[fm][2 * fn][2 * h]) * acc[fm][2 * fn + 1][2 * h]);
                        hi = to_storage<DT>(silu(acc[fm][2 * fn][2 * h + 1]) * acc[fm][2 * fn + 1][2 * h + 1]);
                    }
                } else {
                    float v0 = acc[fm][fn][2 * h], v1 = acc[fm][fn][2 * h + 1];
                    if (act == ACT_GELU_TANH) {
                        v0 = gelu_tanh(v0);
                        v1 = gelu_tanh(v1);
                    }
                    lo = to_storage<DT>(v0);
                    hi = to_storage<DT>(v1);
                }
                pk[fm][fn][h] = lo | (hi << 16);
            }
#pragma unroll
    for (int pass = 0; pass < C::EPI_PASSES; ++pass) {
        const int r0 = pass * C::EPI_ROWS;
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int rbase = wm * C::WTM + fm * 16;          // wave-uniform
            if (rbase < r0 || rbase >= r0 + C::EPI_ROWS) continue;
            const int nf = inter ? NV / 2 : NV;
#pragma unroll
            for (int fn = 0; fn < NV; ++fn) {
                if (fn >= nf) continue;
                const int col = inter ? (wn * C::WTN + 2 * fn * 16) / 2 + (lane & 15)
                                      : wn * C::WTN + fn * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = rbase - r0 + (lane >> 4) * 4 + i;
                    s[row * LD + col] = (uint16_t)(pk[fm][fn][i >> 1] >> (16 * (i & 1)));
                }
            }
        }
        lds_barrier();
        for (int q = thread_index(); q < C::EPI_ROWS * cpr; q += C::NT) {
            const int row = q / cpr, c = q % cpr;
            const int gm = m0 + r0 + row, gn = n0 + c * 8;
            if (gm < rows && gn < cols) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(s + row * LD + c * 8);
                st16(D + (size_t)gm * ldd + gn, v);
            }
        }
        lds_barrier();     // the staging area is free again
    }
}

struct NoWait {
    __device__ __forceinline__ void operator()(int) const {}
};

// Output width of a GEMM1 (producer) tile: BN, or BN/2 for SwiGLU.
template <class C>
__device__ __forceinline__ int producer_width(const ChainArgs& a) {
    return a.act == ACT_SWIGLU ? C::BN / 2 : C::BN;
}

// K-slab range of part s of a tile split into S parts of ksp slabs.
__device__ __forceinline__ void part_range(int nks, uint32_t s, uint32_t ksp, int& ks0, int& ks1) {
    ks0 = (int)(s * ksp);
    ks1 = ks0 + (int)ksp;
    if (ks0 > nks) ks0 = nks;
    if (ks1 > nks) ks1 = nks;
}

// Layer l's buffers (l = 0 in a one-layer chain, where they are x, t and
// y): its input, intermediate T_l and output, computed where they are used
// from the kernel arguments (a copy of every layer's pointers held through
// the item would take scalar registers the main loop needs).
__device__ __forceinline__ const uint16_t* layer_input(const ChainArgs& a, uint32_t l) {
    return l == 0 ? a.x : a.ys + (size_t)(l - 1) * a.M * a.ldy;
}
__device__ __forceinline__ uint16_t* layer_t(const ChainArgs& a, uint32_t l) {
    return l == 0 ? a.t : a.t + (size_t)l * a.M * a.ldt;
}
__device__ __forceinline__ uint16_t* layer_output(const ChainArgs& a, uint32_t l) {
    return l + 1 < a.layers ? a.ys + (size_t)l * a.M * a.ldy : a.y;
}

template <class C>
__device__ __forceinline__ TileJob producer_job(const ChainArgs& a, uint32_t mb, uint32_t nb, uint32_t s,
                                                uint32_t l) {
    const bool inter = a.act == ACT_SWIGLU;
    int ks0, ks1;
    part_range((a.H + BK - 1) / BK, s, a.ksp1, ks0, ks1);
    return TileJob{layer_input(a, l), l == 0 ? a.w1 : a.w1s[l], a.zero, l == 0 ? a.ldx : a.ldy, a.M,
                   (int)mb * C::BM, a.ldw1, a.I, (int)nb * producer_width<C>(a), inter ? a.I : 0,
                   a.H, ks0, ks1, inter};
}

template <class C>
__device__ __forceinline__ TileJob consumer_job(const ChainArgs& a, uint32_t mb, uint32_t nb, uint32_t s,
                                                uint32_t l) {
    int ks0, ks1;
    part_range((a.I + BK - 1) / BK, s, a.ksp2, ks0, ks1);
    return TileJob{layer_t(a, l), l == 0 ? a.w2 : a.w2s[l], a.zero, a.ldt, a.M, (int)mb * C::BM, a.ldw2, a.H,
                   (int)nb * C::BN, 0, a.I, ks0, ks1, false};
}

// Split-K for tiles of more than 16 fragments per thread, whose
// accumulators leave no room for a running sum beside them: every part
// stores its accumulators (fp32, in register order so every thread writes
// and later reads its own 16-byte slots) and counts in with an agent-scope
// release; the part that arrives last sets the tile's counter back to zero
// (every part of this execution has counted in, so the next execution
// starts from zero: no host-side generation, and a captured stream-ordered
// graph replays correctly) and replaces the accumulators by the sum of all
// S partials in part order.  Returns true in the last part (which then runs
// the epilogue).  (The ready-word form below was 4% slower on these tiles.)
template <class C>
__device__ __forceinline__ bool split_reduce_release(f32x4 (&acc)[C::FM][C::FN], float* part, uint32_t* cnt,
                                             uint32_t tile, uint32_t s, uint32_t S, uint32_t* s_flag) {
    constexpr int NF = C::FM * C::FN;
    const int tid = thread_index();
    f32x4* base = reinterpret_cast<f32x4*>(part) + (size_t)tile * S * NF * C::NT;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
            base[((size_t)s * NF + fm * C::FN + fn) * C::NT + tid] = acc[fm][fn];
    chaos_delay(tile * 64u + s);
    // every thread's partial happens before thread 0's agent-scope release
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t old = __hip_atomic_fetch_add(cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old + 1u == S;
        if (last) __hip_atomic_store(cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last ? 1u : 0u;
        handoff_acquire();
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(*s_flag) == 0) return false;
    // Sum in part order (p = 0, 1, .., S-1), every term read back from the
    // partials (this part's own included: its stores completed before the
    // release above, and they hold exactly the register values), so the
    // accumulators are free to hold the sum.  Every fragment's load of one
    // part (chunk) is issued before any of them is used: a part costs one or
    // two memory latencies, not one per fragment.
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = base[(size_t)(fm * C::FN + fn) * C::NT + tid];
    // (in row chunks of at most 16 fragments, so the loaded values take at
    // most 64 registers beside the accumulators)
    constexpr int RC = 16 / C::FN < 1 ? 1 : (16 / C::FN < C::FM ? 16 / C::FN : C::FM);
    static_assert(C::FM % RC == 0, "row chunks");
    for (uint32_t p = 1; p < S; ++p) {
        const f32x4* src = base + (size_t)p * NF * C::NT + tid;
#pragma unroll
        for (int r0 = 0; r0 < C::FM; r0 += RC) {
            f32x4 v[RC][C::FN];
#pragma unroll
            for (int fm = 0; fm < RC; ++fm)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn) v[fm][fn] = src[(size_t)((r0 + fm) * C::FN + fn) * C::NT];
#pragma unroll
            for (int fm = 0; fm < RC; ++fm)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn) acc[r0 + fm][fn] = acc[r0 + fm][fn] + v[fm][fn];
        }
    }
    return true;
}

// Split-K for tiles of at most 16 fragments per thread.  Every part first
// counts in (relaxed atomic add on the tile's counter); the part that
// brings the count to S is the reducing part and
// sets the counter back to zero (every part of this execution has counted
// in, so the next execution starts from zero: no host-side generation, and a
// captured stream-ordered graph replays correctly).  Each other part stores
// its accumulators (fp32, in register order so every thread writes and the
// reducing part's same thread reads its own 16-byte slots), releases them at
// agent scope (the L2 write-back that makes them visible to any XCD) and
// sets its ready word.  The reducing part waits for the S-1 ready words
// (those parts have counted in, so they are running and publish without
// waiting on anything), sets them back to zero, and sums all S partials in
// part order with its own accumulators in their place: the same values in
// the same order as summing S stored partials, so every policy and split
// placement gives the same bits.  Only S-1 parts per tile store and write
// back, and the reducing part never does.  Returns true in the reducing
// part (which then runs the epilogue).  The publishing parts finish within
// a few microseconds of each other, so the reducing part polls at most
// every 4 x 64 clocks.
constexpr uint32_t READY_POLL_MAX_UNITS = 4;

template <class C>
__device__ __forceinline__ bool split_reduce(f32x4 (&acc)[C::FM][C::FN], float* part, uint32_t* cnt, uint32_t* rdy,
                                             uint32_t tile, uint32_t s, uint32_t S, uint32_t* s_flag,
                                             uint32_t* status, uint32_t limit) {
    constexpr int NF = C::FM * C::FN;
    if constexpr (NF > 16) {
        (void)rdy; (void)status; (void)limit;
        return split_reduce_release<C>(acc, part, cnt, tile, s, S, s_flag);
    }
    const int tid = thread_index();
    f32x4* base = reinterpret_cast<f32x4*>(part) + (size_t)tile * S * NF * C::NT;
    uint32_t* ready = rdy + (size_t)tile * S;
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old + 1u == S;
        if (last) __hip_atomic_store(cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last ? 1u : 0u;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(*s_flag) == 0) {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
                base[((size_t)s * NF + fm * C::FN + fn) * C::NT + tid] = acc[fm][fn];
        chaos_delay(tile * 64u + s);
        // every thread's partial happens before thread 0's agent-scope release
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_store(ready + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return false;
    }
    if ((tid >> 6) == 0) {
        // wave 0: lane p waits for part p's ready word (p != s), with back-off;
        // gives up only if the watchdog fires (status records it)
        const uint32_t p = tid & 63;
        const bool mine = p < S && p != s;
        uint32_t polls = 0, units = 1;
        for (;;) {
            const bool ok = !mine || __hip_atomic_load(ready + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
            if (__ballot(!ok) == 0) break;
            if (++polls >= limit || atomic_load_relaxed(status) != 0) {
                if (tid == 0) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            for (uint32_t i = 0; i < units; ++i) __builtin_amdgcn_s_sleep(1);
            if (units < READY_POLL_MAX_UNITS) units <<= 1;
        }
        if (mine) __hip_atomic_store(ready + p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        handoff_acquire();
    }
    __syncthreads();
    // Sum in part order (p = 0, 1, .., S-1), in row groups of at most 8
    // fragments.  The loads of PB parts are all issued before any of them is
    // added, so a reduction over S parts waits for about S / PB memory
    // latencies instead of S - 1 (part by part, the four-part reductions of
    // 16 x 128 tiles spent ~3 us here).  Tiles of at most 8 fragments per
    // thread load up to 16 fragments at once (64 registers beside the
    // accumulators and the running sum); larger ones, whose registers are
    // scarcer, one part at a time.  The additions keep part order, so the
    // bits do not change.
    constexpr int GR = 8 / C::FN < 1 ? 1 : (8 / C::FN < C::FM ? 8 / C::FN : C::FM);
    constexpr int GF = GR * C::FN;
    constexpr int INFLIGHT = NF <= 8 ? 16 : 8;
    constexpr int PB = INFLIGHT / GF < 1 ? 1 : INFLIGHT / GF;
    static_assert(C::FM % GR == 0, "row groups");
#pragma unroll
    for (int r0 = 0; r0 < C::FM; r0 += GR) {
        f32x4 sum[GR][C::FN];
        for (uint32_t p0 = 0; p0 < S; p0 += PB) {
            f32x4 v[PB][GR][C::FN];
#pragma unroll
            for (int b = 0; b < PB; ++b) {
                const uint32_t p = p0 + b;
                if (p < S && p != s) {
                    const f32x4* src = base + (size_t)p * NF * C::NT + tid;
#pragma unroll
                    for (int r = 0; r < GR; ++r)
#pragma unroll
                        for (int fn = 0; fn < C::FN; ++fn) v[b][r][fn] = src[(size_t)((r0 + r) * C::FN + fn) * C::NT];
                }
            }
#pragma unroll
            for (int b = 0; b < PB; ++b) {
                const uint32_t p = p0 + b;
                if (p < S) {
#pragma unroll
                    for (int r = 0; r < GR; ++r)
#pragma unroll
                        for (int fn = 0; fn < C::FN; ++fn) {
                            const f32x4 x = p == s ? acc[r0 + r][fn] : v[b][r][fn];
                            sum[r][fn] = p == 0 ? x : sum[r][fn] + x;
                        }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < GR; ++r)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) acc[r0 + r][fn] = sum[r][fn];
    }
    return true;
}

// One tile part of either GEMM.  ROLE 1 = producer (X W1 -> act -> T),
// 2 = consumer (T W2 -> Y); `wait` is only exercised by consumers.  The role
// is a template parameter so that each role gets its own main loop compiled
// for it (the persistent kernel holds both): with one loop shared at run
// time, the tiles ran 2-20% slower than the same tiles in the stand-alone
// kernels.  Returns true if this part wrote the tile's output (always,
// unless the tile is split and another part arrives last).
struct NoPrefetch {
    __device__ __forceinline__ void operator()() const {}
};

// `done()` is called once the part has no wait left (after its K loop and
// any split-K reduction), before the epilogue: the persistent kernels start
// drawing their next item there, so that the draw overlaps the stores.
template <class C, int DT, int ROLE, class Wait, class Done = NoPrefetch>
__device__ __forceinline__ bool run_tile(const ChainArgs& a, uint32_t mb, uint32_t nb, uint32_t s, uint32_t* s_flag,
                                         Wait& wait, uint32_t l = 0, Done done = Done{}) {
    f32x4 acc[C::FM][C::FN];
    // layer l's split-K counters, ready words and partials follow layer
    // l-1's: its tiles are numbered from l * T1 (GEMM1) or l * T2 (GEMM2)
    const uint32_t tile = (ROLE == 1 ? l * a.T1 + mb * a.N1t : l * a.T2 + mb * a.N2t) + nb;
    const TileJob j = ROLE == 1 ? producer_job<C>(a, mb, nb, s, l) : consumer_job<C>(a, mb, nb, s, l);
    tile_mainloop<C, DT>(j, acc, wait);
    // timeline: a GEMM1 part's second word is the end of its K loop
    if (ROLE == 1 && l == 0 && a.trace && thread_index() == 0)
        a.trace[4 * (size_t)((mb * a.N1t + nb) * a.S1 + s) + 1] = __builtin_amdgcn_s_memrealtime();
    const uint32_t S = ROLE == 1 ? a.S1 : a.S2;
    if (S > 1) {
        const bool last = ROLE == 1 ? split_reduce<C>(acc, a.part1, a.cnt1, a.rdy1, tile, s, S, s_flag, a.status, a.spin_limit)
                                    : split_reduce<C>(acc, a.part2, a.cnt2, a.rdy2, tile, s, S, s_flag, a.status, a.spin_limit);
        done();
        if (!last) return false;
    } else {
        done();
    }
    if constexpr (ROLE == 1)
        tile_epilogue<C, DT>(acc, a.act, j.inter, layer_t(a, l), a.ldt, a.M, a.I, j.m0, j.n0);
    else
        tile_epilogue<C, DT>(acc, ACT_NONE, false, layer_output(a, l), l + 1 < a.layers ? a.ldy : a.ldo, a.M, a.H,
                             j.m0, j.n0);
    return true;
}

}  // namespace mlpc
