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

// One workgroup per tile part: blockIdx = tile * S + part.
template <class C, int DT>
__global__ __launch_bounds__(C::NT) void gemm1_act_kernel(ChainArgs a) {
    __shared__ uint32_t s_flag;
    NoWait w;
    run_tile<C, DT>(a, 1, blockIdx.x / a.S1, blockIdx.x % a.S1, &s_flag, w);
}

template <class C, int DT>
__global__ __launch_bounds__(C::NT) void gemm2_kernel(ChainArgs a) {
    __shared__ uint32_t s_flag;
    NoWait w;
    run_tile<C, DT>(a, 2, blockIdx.x / a.S2, blockIdx.x % a.S2, &s_flag, w);
}

// Consumer-side wait of the persistent kernel.  One functor type serves
// producer tiles (inactive) and consumer tiles, so the kernel holds a single
// inlined copy of the tile main loop.  Only wave 0 polls and takes the
// acquire fence; the result reaches the other waves through LDS behind a
// barrier that leaves the DMA ring in flight, so one L2 invalidation covers
// the whole workgroup.
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
    uint32_t* s_ready;       // LDS broadcast slot
    uint32_t ready;          // tile_sync: blocks below this are acquired or not needed (uniform)
    bool waited;             // row_sync: the part's single wait is done (uniform)
    __device__ __forceinline__ void operator()(int ks) {
        if (!active) return;
        if constexpr (POL == POL_ROW) {
            if (waited) return;
            waited = true;
            if ((threadIdx.x >> 6) == 0) wave_acquire_count(cnt, target, status, limit);
            lds_barrier();
        } else {
            uint32_t need = (uint32_t)((ks * BK + BK - 1) / bn1);    // last block slab ks reads
            if (need > n1t - 1) need = n1t - 1;
            if (need < ready) return;
            if ((threadIdx.x >> 6) == 0) {
                const uint32_t r = wave_acquire_flags(flags, ready, need, n1t, target, status, limit);
                if (threadIdx.x == 0) *s_ready = r;
            }
            lds_barrier();
            ready = __builtin_amdgcn_readfirstlane(*s_ready);
        }
    }
};

template <class C, int DT, int POL>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC)))
void chain_persistent_kernel(ChainArgs a) {
    __shared__ uint32_t s_ticket;
    __shared__ uint32_t s_ready;
    __shared__ uint32_t s_flag;
    // tickets [0, P1) are GEMM1 tile parts, [P1, P1 + P2) GEMM2 tile parts
    const uint32_t P1 = a.T1 * a.S1, P2 = a.T2 * a.S2;
    const uint32_t total = P1 + P2;
    const int bn1 = a.act == ACT_SWIGLU ? C::BN / 2 : C::BN;
    for (;;) {
        if (threadIdx.x == 0)
            s_ticket = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                       a.ticket_base;
        __syncthreads();
        // The ticket is the same for every thread of the workgroup; reading it
        // through readfirstlane makes that visible to the compiler, so every
        // branch on it (and the loop exit) is a scalar branch and all lanes of
        // a wave stay on one path through the barriers below.
        const uint32_t t = __builtin_amdgcn_readfirstlane(s_ticket);
        __syncthreads();
        if (t >= total) break;
        const bool prod = t < P1;
        // test hook: a skipped producer part does no work and no release
        if (!(prod && t == a.skip_producer)) {
            const uint32_t S = prod ? a.S1 : a.S2;
            const uint32_t u = prod ? t : t - P1;
            const uint32_t tile = u / S, part = u % S;
            uint32_t mb, nb;
            tile_coords(tile, a.Mt, prod ? a.N1t : a.N2t, a.group_m, mb, nb);
            // first producer block the part's K range reads
            const uint32_t first = prod ? 0u : (part * a.ksp2 * BK) / (uint32_t)bn1;
            ChainWait<POL> w{!prod, a.flags + mb * a.N1t, a.rowcnt + mb, a.N1t,
                             POL == POL_ROW ? a.epoch * a.N1t : a.epoch, bn1, a.status, a.spin_limit,
                             &s_ready, first, false};
            const bool wrote = run_tile<C, DT>(a, prod ? 1 : 2, tile, part, &s_flag, w);
            if (prod && wrote) {
                // every thread's T stores happen before thread 0's agent-scope
                // release (workgroup release + barrier), which publishes the tile
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                __syncthreads();
                if (threadIdx.x == 0) {
                    if constexpr (POL == POL_TILE)
                        __hip_atomic_store(a.flags + mb * a.N1t + nb, a.epoch, __ATOMIC_RELEASE,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    else
                        __hip_atomic_fetch_add(a.rowcnt + mb, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        // Keep this barrier: it separates the thread-0-only release above from
        // the thread-0-only ticket draw at the top of the loop.  Without it the
        // compiler may merge the two across the back edge into a loop in which
        // the other threads re-read the old ticket at the barriers while
        // thread 0 waits to draw the next one, which never ends.
        __syncthreads();
    }
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
    default:
        return hipErrorInvalidValue;
    }
}

template <class C>
static hipError_t launch_c(const ChainArgs& a, int dtype, int what, int grid, hipStream_t s, int* occ) {
    return dtype == DT_F16 ? launch_t<C, DT_F16>(a, what, grid, s, occ)
                           : launch_t<C, DT_BF16>(a, what, grid, s, occ);
}

#define MLPC_PICK(id, bm, bn, wm, wn, ns, occ) \
    if constexpr (id == MLPC_CFG) return TileCfg<bm, bn, wm, wn, ns, occ>{};
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

hipError_t MLPC_CAT(mlpc_occupancy_cfg, MLPC_CFG)(int dtype, int policy, int* per_cu) {
    ChainArgs dummy{};
    return launch_c<Cfg>(dummy, dtype, policy == POL_ROW ? LAUNCH_ROW : LAUNCH_TILE, 0, nullptr, per_cu);
}

CfgInfo MLPC_CAT(mlpc_info_cfg, MLPC_CFG)() {
    return CfgInfo{MLPC_CFG, Cfg::BM, Cfg::BN, BK, Cfg::NT, Cfg::lds_bytes()};
}
