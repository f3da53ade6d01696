// chain_kernels.hip -- the kernels of the MLP GEMM chain and their launchers.
//
//   gemm1_act_kernel   one workgroup per GEMM1 tile: X W1 -> act -> T
//   gemm2_kernel       one workgroup per GEMM2 tile: T W2 -> Y
//   chain_persistent   one workgroup per CU slot, looping over an atomic tile
//                      queue that hands out every GEMM1 (producer) tile before
//                      any GEMM2 (consumer) tile.  A consumer only ever waits
//                      for producers whose tickets were drawn earlier by
//                      running workgroups, and producers never wait, so every
//                      wait ends whatever the grid size.
//
// The stream-ordered policy is the first two kernels back to back on one
// stream (kernel-level dependency); row_sync and tile_sync are the
// persistent kernel with per-row-block counters or per-tile flags
// (tile-level dependency, as in the CuSync README's opening paragraph and the
// megakernel discussion in the Hacker News thread on megakernels vs CUDA
// graphs, where a consumer task starts as soon as its slice is done).
//
// This file is compiled once per tile configuration (MLPC_CFG = the id in
// chain_configs.h); each object defines the launchers of that configuration.
#include "chain_configs.h"
#include "chain_device.hpp"
#include "chain_launch.h"

#ifndef MLPC_CFG
#error "compile with -DMLPC_CFG=<configuration id>"
#endif

namespace mlpc {

// Timeline record of item t (thread 0): start, end of its last wait (a
// GEMM1 part of a one-layer run: end of its K loop, written by run_tile;
// t_waited = ~0 keeps it), end (100 MHz realtime clock), and where it ran.
__device__ __forceinline__ void trace_item(const ChainArgs& a, uint32_t t, uint64_t t_start, uint64_t t_waited,
                                           bool wrote) {
    uint32_t hw = 0, xcc = 0;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    uint64_t* r = a.trace + 4 * (size_t)t;
    r[0] = t_start;
    if (t_waited != ~0ull) r[1] = t_waited;
    r[2] = __builtin_amdgcn_s_memrealtime();
    r[3] = (uint64_t)t | ((uint64_t)(xcc & 0xf) << 32) | ((uint64_t)hw << 36) | ((uint64_t)wrote << 63);
}

// One workgroup per tile part.  Workgroups are dispatched to the XCDs
// round-robin, so block b runs on XCD b % 8: give each XCD a contiguous
// chunk of the concatenated XCD blocks.
template <class C, int DT>
__global__ __launch_bounds__(C::NT) void gemm1_act_kernel(ChainArgs a) {
    __shared__ uint32_t s_flag;
    NoWait w;
    uint32_t mb, nb, part;
    xcd_position(a.Mt, a.N1t, a.S1, a.rx, a.order & 1u, xcd_chunked(blockIdx.x, a.T1 * a.S1), mb, nb, part);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const bool wrote = run_tile<C, DT, 1>(a, mb, nb, part, &s_flag, w);
    if (a.trace && threadIdx.x == 0) trace_item(a, (mb * a.N1t + nb) * a.S1 + part, t0, ~0ull, wrote);
}

template <class C, int DT>
__global__ __launch_bounds__(C::NT) void gemm2_kernel(ChainArgs a) {
    __shared__ uint32_t s_flag;
    NoWait w;
    uint32_t mb, nb, part;
    xcd_position(a.Mt, a.N2t, a.S2, a.rx, (a.order >> 1) & 1u, xcd_chunked(blockIdx.x, a.T2 * a.S2), mb, nb, part);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const bool wrote = run_tile<C, DT, 2>(a, mb, nb, part, &s_flag, w);
    if (a.trace && threadIdx.x == 0)
        trace_item(a, a.T1 * a.S1 + (mb * a.N2t + nb) * a.S2 + part, t0, t0, wrote);
}

// Consumer-side wait of the persistent kernel.  Only wave 0 polls and takes
// the hand-off acquire (handoff_acquire); the result reaches the other waves
// through LDS behind a barrier that leaves the DMA ring in flight, and every
// wave's later operand loads follow that barrier.
//   row_sync:  before the first slab of the part, wait until all N1t
//              producer tiles of the row block have counted themselves in
//              for this epoch;
//   tile_sync: before slab ks, make sure every producer column block that
//              slab reads has been acquired; if not, wave 0 waits for it and
//              acquires every block that is ready by then in one go.  A part
//              starts at the first block of its own K range.  Slabs are
//              still taken in ascending K order.
template <int POL>
struct ChainWait {
    bool active;             // consumer tile (uniform)
    const uint32_t* flags;   // tile_sync: the row block's N1t flags
    const uint32_t* cnt;     // row_sync: the row block's counter
    uint32_t n1t;
    uint32_t target;         // tile_sync: epoch; row_sync: epoch * N1t
    int bn1;                 // output columns per producer tile
    uint32_t* status;
    uint32_t limit;
    uint32_t agent;          // hand-offs invalidate the L2 (producer tiles share lines of T)
    uint32_t* s_ready;       // LDS broadcast slot
    uint32_t ready;          // tile_sync: blocks below this are acquired or not needed (uniform)
    bool waited;             // row_sync: the part's single wait is done (uniform)
    uint64_t t_waited;       // realtime clock after the last wait (timeline trace)
    __device__ __forceinline__ void operator()(int ks) {
        if (!active) return;
        if constexpr (POL == POL_ROW) {
            if (waited) return;
            waited = true;
            if ((threadIdx.x >> 6) == 0) wave_acquire_count(cnt, target, status, limit, agent);
            lds_barrier();
            t_waited = __builtin_amdgcn_s_memrealtime();
        } else {
            uint32_t need = (uint32_t)((ks * BK + BK - 1) / bn1);    // last block slab ks reads
            if (need > n1t - 1) need = n1t - 1;
            if (need < ready) return;
            if ((threadIdx.x >> 6) == 0) {
                const uint32_t r = wave_acquire_flags(flags, ready, need, n1t, target, status, limit, agent);
                if (threadIdx.x == 0) *s_ready = r;
            }
            lds_barrier();
            ready = __builtin_amdgcn_readfirstlane(*s_ready);
            t_waited = __builtin_amdgcn_s_memrealtime();
        }
    }
};

// The tile queues.  Queue x (one per XCD) holds the GEMM1 tile parts of XCD
// x's block of the GEMM1 grid, then the GEMM2 tile parts of its block of the
// GEMM2 grid (same row split), each walked row-major.  Workgroup b belongs to
// queue b % 8 -- the XCD it is dispatched to -- and starts with item b / 8
// of it, with no atomic (queue x's first items, one per owner, are handed
// out at launch).  Further items are drawn by wave 0: one round of relaxed
// loads reads the counters of all queues not yet seen dry, and an atomic
// draws from the first of them, in the order own queue, then the next ones
// -- so a workgroup takes its own queue's remaining items before stealing.
// Runs alternate between two sets of counters (epoch parity): workgroup 0
// zeroes the set the previous run used, which the next run takes, so every
// run starts from zero with no clearing launch (stream order: the previous
// run has finished, and this one never touches that set).  Items are numbered for
// flags, trace and test hooks as GEMM1 parts (mb * N1t + nb) * S1 + part,
// then GEMM2 parts P1 + (mb * N2t + nb) * S2 + part.
// Deadlock freedom: a queue hands out its items in order, producers first,
// so a consumer is handed out only after every producer of its queue has
// been; a consumer waits only for producers; every queue has an owner (grid
// >= 8), and an owner takes its own queue's items before any other's, so a
// producer not yet handed out will be, by an owner that is running a
// producer or about to draw one -- producers never wait.
struct Queues {
    uint32_t own;
    uint32_t dry;          // bit v: queue (own + v) & 7 is known to be empty (wave-uniform)
    uint32_t P1;
    uint32_t* ticket;      // this run's set of 8 queue counters
};

__device__ __forceinline__ uint32_t queue_item(const ChainArgs& a, const XcdBlock& bp, const XcdBlock& bc,
                                               uint32_t P1, uint32_t c) {
    uint32_t mb, nb, part;
    if (c < bp.len) {
        xcd_item(bp, a.S1, a.order & 1u, c, mb, nb, part);
        return (mb * a.N1t + nb) * a.S1 + part;
    }
    xcd_item(bc, a.S2, (a.order >> 1) & 1u, c - bp.len, mb, nb, part);
    return P1 + (mb * a.N2t + nb) * a.S2 + part;
}

// Owners of queue x: workgroups b < grid with b % 8 == x.
__device__ __forceinline__ uint32_t queue_owners(uint32_t grid, uint32_t x) {
    return grid > x ? (grid - x + 7) / 8 : 0;
}

// Item c of queue (bp, bc) of a chain of a.layers MLP layers: queue order
// is layer by layer (each layer's GEMM1 parts, then its GEMM2 parts), and
// layer l's items are numbered from l * (P1 + P2).
__device__ __forceinline__ uint32_t queue_item_layers(const ChainArgs& a, const XcdBlock& bp, const XcdBlock& bc,
                                                      uint32_t P1, uint32_t c) {
    const uint32_t per = bp.len + bc.len;
    const uint32_t l = c / per;
    return l * (P1 + a.T2 * a.S2) + queue_item(a, bp, bc, P1, c - l * per);
}

// Wave 0 only: the next item for this workgroup, or NO_ITEM.
constexpr uint32_t NO_ITEM = 0xffffffffu;
template <bool LAYERS = false>
__device__ __forceinline__ uint32_t draw_item(const ChainArgs& a, Queues& q) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t x = (q.own + lane) & 7;
    XcdBlock bp{0, 0, 1, 1, 0}, bc{0, 0, 1, 1, 0};
    uint32_t len = 0, first = 0;
    if (lane < 8) {
        bp = xcd_block(a.Mt, a.N1t, a.S1, a.rx, x);
        bc = xcd_block(a.Mt, a.N2t, a.S2, a.rx, x);
        len = (LAYERS ? a.layers : 1u) * (bp.len + bc.len);
        first = min(len, queue_owners(a.grid, x));   // items handed out at launch
    }
    for (;;) {
        bool avail = false;
        if (lane < 8 && !((q.dry >> lane) & 1u))
            avail = atomic_load_relaxed(q.ticket + 64 * x) + first < len;
        const uint64_t m = __ballot(avail);
        if (m == 0) return NO_ITEM;
        const uint32_t k = (uint32_t)__builtin_ctzll(m);
        uint32_t item = NO_ITEM;
        if (lane == k) {
            const uint32_t c = __hip_atomic_fetch_add(q.ticket + 64 * x, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT) + first;
            if (c < len) item = LAYERS ? queue_item_layers(a, bp, bc, q.P1, c) : queue_item(a, bp, bc, q.P1, c);
        }
        item = __builtin_amdgcn_readlane(item, k);
        if (item != NO_ITEM) return item;
        q.dry |= 1u << k;
    }
}

// Publication of a ready flag by wave 0 (called by all its lanes, after the
// workgroup barrier that follows the tile's stores): one agent-scope release,
// then lane x < 8 stores the epoch into XCD x's copy of the flags.
__device__ __forceinline__ void publish_flag(const ChainArgs& a, uint32_t idx, uint32_t epoch) {
    const uint32_t lane = threadIdx.x & 63;
    if (lane < 8) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_store(a.flags + lane * a.fstride + idx, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The epoch of a fused run, kept on the device so that a run depends on
// nothing the host passes per run (a captured graph replays it as is).  A
// 64-bit word counts runs in its high half: every workgroup adds to it once,
// after its last item, and the adds of one run sum to exactly 2^32
// (workgroup 0 adds 2^32 - grid + 1, every other one 1).  A workgroup reads
// the word at launch, before its own add, so at most grid - 1 adds of its
// own run precede the value it reads and the high half is still the count of
// finished runs: the run's epoch is one more.  Only the ordering of accesses
// to this one word is needed (each workgroup's read comes before its own add;
// the next run is ordered after this one by its stream).  The count wraps at
// 2^32 runs like every other epoch comparison.
__device__ __forceinline__ uint32_t run_epoch(const ChainArgs& a) {
    const uint64_t w = __hip_atomic_load(a.run_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane((uint32_t)(w >> 32)) + 1u;
}

// Thread 0 of each workgroup, after its last item: its share of the run
// counter (no result is needed).
__device__ __forceinline__ void run_finished(const ChainArgs& a) {
    if (threadIdx.x == 0) {
        const uint64_t add = blockIdx.x == 0 ? (1ull << 32) - gridDim.x + 1u : 1ull;
        (void)__hip_atomic_fetch_add(a.run_epoch, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Early draw.  Once an item has no wait left (its K loop and split-K
// reduction are done), the first thread of wave 1 takes the next position of
// the own queue with one atomic, and the epilogue's stores and the
// publication run while it is in flight; after the publication it leaves the
// position in LDS, and wave 0 resolves it at the top of the loop
// (resolve_early), falling back to draw_item, which scans the other queues,
// only when that position is past the queue's end.  The draw of the next
// item then costs the workgroup about one memory round trip less (two
// before: the counters' loads, then the atomic).  The atomic is wave 1's so
// that the release that publishes the item (thread 0's) does not wait for it:
// at the end of a wave of producers the queue counters are contended and the
// atomic can take microseconds.  An item never waits for one its own
// workgroup holds: the early draw comes after the current item's last wait.
constexpr uint32_t EARLY_THREAD = 64;

struct EarlyDraw {
    uint32_t* ticket;   // this run's set of queue counters
    uint32_t own;
    bool& issued;       // uniform: an early draw was started for the current item
    uint32_t& pos;      // thread EARLY_THREAD: the position the atomic returned
    __device__ __forceinline__ void operator()() const {
        issued = true;
        // (a wrapping increment with an all-ones bound is +1 here; unlike an
        // atomic add the compiler does not rewrite it into a wave-wide add
        // whose result it waits for at once)
        if (threadIdx.x == EARLY_THREAD)
            pos = __builtin_amdgcn_atomic_inc32(ticket + 64 * own, 0xffffffffu, __ATOMIC_RELAXED, "agent");
    }
};

// Wave 0 only: the item at the position the early draw took, or NO_ITEM
// with the own queue marked dry.
template <bool LAYERS>
__device__ __forceinline__ uint32_t resolve_early(const ChainArgs& a, Queues& q, uint32_t c) {
    if (q.dry & 1u) return NO_ITEM;
    const XcdBlock bp = xcd_block(a.Mt, a.N1t, a.S1, a.rx, q.own);
    const XcdBlock bc = xcd_block(a.Mt, a.N2t, a.S2, a.rx, q.own);
    const uint32_t len = (LAYERS ? a.layers : 1u) * (bp.len + bc.len);
    const uint32_t p = c + min(len, queue_owners(a.grid, q.own));
    if (p < len) return LAYERS ? queue_item_layers(a, bp, bc, q.P1, p) : queue_item(a, bp, bc, q.P1, p);
    q.dry |= 1u;
    return NO_ITEM;
}

template <class C, int DT, int POL>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC)))
void chain_persistent_kernel(ChainArgs a) {
    __shared__ uint32_t s_ticket;
    __shared__ uint32_t s_ready;
    __shared__ uint32_t s_flag;
    __shared__ uint32_t s_pos;
    const uint32_t P1 = a.T1 * a.S1;
    const int bn1 = a.act == ACT_SWIGLU ? C::BN / 2 : C::BN;
    const uint32_t epoch = run_epoch(a);
    Queues q{blockIdx.x & 7u, 0u, P1, a.ticket + 512 * (epoch & 1u)};
    uint32_t item = NO_ITEM;
    if (blockIdx.x == 0 && threadIdx.x < 8)
        __hip_atomic_store(a.ticket + 512 * ((epoch & 1u) ^ 1u) + 64 * threadIdx.x, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    {
        // the launch-time item: position blockIdx / 8 of the own queue
        const XcdBlock bp = xcd_block(a.Mt, a.N1t, a.S1, a.rx, q.own);
        const XcdBlock bc = xcd_block(a.Mt, a.N2t, a.S2, a.rx, q.own);
        const uint32_t pos = blockIdx.x >> 3;
        if (pos < bp.len + bc.len) item = queue_item(a, bp, bc, P1, pos);
    }
    bool issued = false;
    uint32_t pos = 0;
    static_assert(C::NT > EARLY_THREAD, "the early draw is wave 1's");
    const EarlyDraw early{q.ticket, q.own, issued, pos};
    for (;;) {
        if (item == NO_ITEM) {
            // the next item (wave 0): the early draw's, else from the own
            // queue or the next ones
            if ((threadIdx.x >> 6) == 0) {
                uint32_t it = issued ? resolve_early<false>(a, q, s_pos) : NO_ITEM;
                if (it == NO_ITEM) it = draw_item(a, q);
                if (threadIdx.x == 0) s_ticket = it;
            }
            issued = false;
            __syncthreads();
            // The item is the same for every thread of the workgroup; reading
            // it through readfirstlane makes that visible to the compiler, so
            // every branch on it (and the loop exit) is a scalar branch and
            // all lanes of a wave stay on one path through the barriers below.
            item = __builtin_amdgcn_readfirstlane(s_ticket);
            __syncthreads();
            if (item == NO_ITEM) break;
        }
        const uint32_t t = item;
        item = NO_ITEM;
        const bool prod = t < P1;
        // test hook: a skipped producer part does no work and no release
        if (!(prod && t == a.skip_producer)) {
            const uint32_t S = prod ? a.S1 : a.S2;
            const uint32_t u = prod ? t : t - P1;
            const uint32_t tile = u / S, part = u % S;
            const uint32_t nt = prod ? a.N1t : a.N2t;
            const uint32_t mb = tile / nt, nb = tile % nt;
            // first producer block the part's K range reads
            const uint32_t first = prod ? 0u : (part * a.ksp2 * BK) / (uint32_t)bn1;
            const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
            ChainWait<POL> w{!prod, a.flags + q.own * a.fstride + mb * a.N1t, a.rowcnt + mb, a.N1t,
                             prod ? 0u : POL == POL_ROW ? epoch * a.N1t : epoch, bn1, a.status, a.spin_limit,
                             a.acq_agent, &s_ready, first, false, t_start};
            bool wrote;
            if (prod) {
                NoWait nw;
                wrote = run_tile<C, DT, 1>(a, mb, nb, part, &s_flag, nw, 0, early);
            } else {
                wrote = run_tile<C, DT, 2>(a, mb, nb, part, &s_flag, w, 0, early);
            }
            if (a.trace && threadIdx.x == 0) trace_item(a, t, t_start, prod ? ~0ull : w.t_waited, wrote);
            if (prod && wrote) {
                chaos_delay(t ^ (epoch << 20));
                // every thread's T stores happen before thread 0's agent-scope
                // release (workgroup release + barrier), which publishes the tile
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                __syncthreads();
                if constexpr (POL == POL_TILE) {
                    if ((threadIdx.x >> 6) == 0) publish_flag(a, mb * a.N1t + nb, epoch);
                } else if (threadIdx.x == 0) {
                    __hip_atomic_fetch_add(a.rowcnt + mb, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if (issued && threadIdx.x == EARLY_THREAD) s_pos = pos;
        // Keep this barrier: it separates the thread-0-only release above from
        // the thread-0-only ticket draw at the top of the loop.  Without it the
        // compiler may merge the two across the back edge into a loop in which
        // the other threads re-read the old ticket at the barriers while
        // thread 0 waits to draw the next one, which never ends.
        __syncthreads();
    }
    run_finished(a);
}

// Persistent kernel of a chain of a.layers MLP layers, 2 * layers dependent
// GEMMs in one launch: layer l's GEMM2 tiles wait for the GEMM1 tiles of T_l
// they read (as in the one-layer kernel), and layer l+1's GEMM1 tiles wait,
// K chunk by K chunk, for the GEMM2 tiles of Y_l they read -- so the
// consumers of one layer overlap the tail of the previous one, which a
// sequence of kernels (or a captured graph of them) cannot do (the Hacker
// News thread on megakernels vs CUDA graphs: one task starts as soon as the
// slice it needs is done, across layers).  Every GEMM output but the last
// publishes per-tile flags (tile_sync) or per-row-block counts (row_sync):
// T_l's at flags + l T1 / rowcnt + l Mt, Y_l's at flags + layers T1 + l T2 /
// rowcnt + (layers + l) Mt.  The queues hand out each XCD's items layer by
// layer, producers before consumers within a layer, so every item an item
// waits for was handed out before it; with every queue owned by a resident
// workgroup that drains its own queue first, every wait ends (the item of
// lowest layer and stage among the waiting ones waits on an item that is
// running and does not wait, or on one its queue's owners will draw).
template <class C, int DT, int POL>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC)))
void chain_layers_kernel(ChainArgs a) {
    __shared__ uint32_t s_ticket;
    __shared__ uint32_t s_ready;
    __shared__ uint32_t s_flag;
    __shared__ uint32_t s_pos;
    const uint32_t P1 = a.T1 * a.S1;
    const uint32_t P = P1 + a.T2 * a.S2;      // items per layer
    const int bn1 = a.act == ACT_SWIGLU ? C::BN / 2 : C::BN;
    const uint32_t epoch = run_epoch(a);
    Queues q{blockIdx.x & 7u, 0u, P1, a.ticket + 512 * (epoch & 1u)};
    uint32_t item = NO_ITEM;
    if (blockIdx.x == 0 && threadIdx.x < 8)
        __hip_atomic_store(a.ticket + 512 * ((epoch & 1u) ^ 1u) + 64 * threadIdx.x, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    {
        const XcdBlock bp = xcd_block(a.Mt, a.N1t, a.S1, a.rx, q.own);
        const XcdBlock bc = xcd_block(a.Mt, a.N2t, a.S2, a.rx, q.own);
        const uint32_t pos = blockIdx.x >> 3;
        if (pos < a.layers * (bp.len + bc.len)) item = queue_item_layers(a, bp, bc, P1, pos);
    }
    bool issued = false;
    uint32_t pos = 0;
    static_assert(C::NT > EARLY_THREAD, "the early draw is wave 1's");
    const EarlyDraw early{q.ticket, q.own, issued, pos};
    for (;;) {
        if (item == NO_ITEM) {
            if ((threadIdx.x >> 6) == 0) {
                uint32_t it = issued ? resolve_early<true>(a, q, s_pos) : NO_ITEM;
                if (it == NO_ITEM) it = draw_item<true>(a, q);
                if (threadIdx.x == 0) s_ticket = it;
            }
            issued = false;
            __syncthreads();
            item = __builtin_amdgcn_readfirstlane(s_ticket);
            __syncthreads();
            if (item == NO_ITEM) break;
        }
        const uint32_t t = item;
        item = NO_ITEM;
        const uint32_t l = t / P, u = t - l * P;
        const bool prod = u < P1;
        if (t != a.skip_producer) {
            const uint32_t S = prod ? a.S1 : a.S2;
            const uint32_t v = prod ? u : u - P1;
            const uint32_t tile = v / S, part = v % S;
            const uint32_t nt = prod ? a.N1t : a.N2t;
            const uint32_t mb = tile / nt, nb = tile % nt;
            const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
            uint64_t t_waited = t_start;
            bool wrote;
            if (prod) {
                // GEMM1 of layer l > 0 reads Y_{l-1}: its K chunks are Y's
                // column blocks of BN (whole 128-byte lines per tile); layer
                // 0's GEMM1 reads x and waits for nothing (an inactive wait,
                // so that both share one copy of the tile code)
                const uint32_t lp = l > 0 ? l - 1 : 0;
                const uint32_t* fy = a.flags + q.own * a.fstride + a.layers * a.T1 + lp * a.T2;
                const uint32_t* cy = a.rowcnt + (a.layers + lp) * a.Mt;
                ChainWait<POL> w{l > 0, fy + mb * a.N2t, cy + mb, a.N2t,
                                 l == 0 ? 0u : POL == POL_ROW ? epoch * a.N2t : epoch, C::BN, a.status,
                                 a.spin_limit,
                                 0u, &s_ready, (part * a.ksp1 * BK) / (uint32_t)C::BN, false, t_start};
                wrote = run_tile<C, DT, 1>(a, mb, nb, part, &s_flag, w, l, early);
                t_waited = w.t_waited;
            } else {
                ChainWait<POL> w{true, a.flags + q.own * a.fstride + l * a.T1 + mb * a.N1t, a.rowcnt + l * a.Mt + mb, a.N1t,
                                 POL == POL_ROW ? epoch * a.N1t : epoch, bn1, a.status, a.spin_limit,
                                 a.acq_agent, &s_ready, (part * a.ksp2 * BK) / (uint32_t)bn1, false, t_start};
                wrote = run_tile<C, DT, 2>(a, mb, nb, part, &s_flag, w, l, early);
                t_waited = w.t_waited;
            }
            if (a.trace && threadIdx.x == 0) trace_item(a, t, t_start, t_waited, wrote);
            if (wrote && (prod || l + 1 < a.layers)) {
                // publish the tile of T_l (GEMM1) or Y_l (GEMM2 of a layer that is not the last)
                chaos_delay(t ^ (epoch << 20));
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                __syncthreads();
                if constexpr (POL == POL_TILE) {
                    if ((threadIdx.x >> 6) == 0)
                        publish_flag(a, prod ? l * a.T1 + mb * a.N1t + nb : a.layers * a.T1 + l * a.T2 + mb * a.N2t + nb,
                                     epoch);
                } else if (threadIdx.x == 0) {
                    uint32_t* c = prod ? a.rowcnt + l * a.Mt + mb : a.rowcnt + (a.layers + l) * a.Mt + mb;
                    __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if (issued && threadIdx.x == EARLY_THREAD) s_pos = pos;
        // (as in the one-layer kernel: keeps the thread-0 release apart from
        // the thread-0 ticket draw at the top of the loop)
        __syncthreads();
    }
    run_finished(a);
}

// ------------------------------------------------------------------ host side

template <class C, int DT>
static hipError_t launch_t(const ChainArgs& a, int what, int grid, hipStream_t s, int* occ) {
    // all LDS is static (one object per pipeline stage)
    switch (what) {
    case LAUNCH_GEMM1:
        hipLaunchKernelGGL((gemm1_act_kernel<C, DT>), dim3(a.T1 * a.S1), dim3(C::NT), 0, s, a);
        return hipGetLastError();
    case LAUNCH_GEMM2:
        hipLaunchKernelGGL((gemm2_kernel<C, DT>), dim3(a.T2 * a.S2), dim3(C::NT), 0, s, a);
        return hipGetLastError();
    case LAUNCH_ROW:
    case LAUNCH_TILE: {
        auto k = (what == LAUNCH_ROW) ? chain_persistent_kernel<C, DT, POL_ROW>
                                      : chain_persistent_kernel<C, DT, POL_TILE>;
        if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, k, C::NT, 0);
        hipLaunchKernelGGL(k, dim3(grid), dim3(C::NT), 0, s, a);
        return hipGetLastError();
    }
    case LAUNCH_LAYERS_ROW:
    case LAUNCH_LAYERS_TILE: {
        auto k = (what == LAUNCH_LAYERS_ROW) ? chain_layers_kernel<C, DT, POL_ROW>
                                             : chain_layers_kernel<C, DT, POL_TILE>;
        if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, k, C::NT, 0);
        hipLaunchKernelGGL(k, dim3(grid), dim3(C::NT), 0, s, a);
        return hipGetLastError();
    }
    default:
        return hipErrorInvalidValue;
    }
}

template <class C>
static hipError_t launch_c(const ChainArgs& a, int dtype, int what, int grid, hipStream_t s, int* occ) {
    return dtype == DT_F16 ? launch_t<C, DT_F16>(a, what, grid, s, occ)
                           : launch_t<C, DT_BF16>(a, what, grid, s, occ);
}

#define MLPC_PICK(id, bm, bn, wm, wn, ns, occ, ks) \
    if constexpr (id == MLPC_CFG) return TileCfg<bm, bn, wm, wn, ns, occ, ks>{};
static constexpr auto this_cfg() { MLPC_CONFIGS(MLPC_PICK) }
#undef MLPC_PICK
using Cfg = decltype(this_cfg());

}  // namespace mlpc

using namespace mlpc;

#define MLPC_CAT2(a, b) a##b
#define MLPC_CAT(a, b) MLPC_CAT2(a, b)

hipError_t MLPC_CAT(mlpc_launch_cfg, MLPC_CFG)(const ChainArgs& a, int dtype, int what, int grid, hipStream_t s) {
    return launch_c<Cfg>(a, dtype, what, grid, s, nullptr);
}

hipError_t MLPC_CAT(mlpc_occupancy_cfg, MLPC_CFG)(int dtype, int policy, int layers, int* per_cu) {
    ChainArgs dummy{};
    const int what = layers > 1 ? (policy == POL_ROW ? LAUNCH_LAYERS_ROW : LAUNCH_LAYERS_TILE)
                                : (policy == POL_ROW ? LAUNCH_ROW : LAUNCH_TILE);
    return launch_c<Cfg>(dummy, dtype, what, 0, nullptr, per_cu);
}

CfgInfo MLPC_CAT(mlpc_info_cfg, MLPC_CFG)() {
    return CfgInfo{MLPC_CFG, Cfg::BM, Cfg::BN, BK, Cfg::NT, Cfg::lds_bytes()};
}
