// chain_api.cpp -- the C ABI declared in include/mlp_chain.h: argument
// checks, tile planning, workspace ownership, epochs and launches.
//
// Per-run synchronization state lives in the workspace and is never cleared
// from the host between runs (no memset on the run path, so a run is a
// single kernel for the fused policies):
//   * a fused run's epoch is kept on the device: a 64-bit word counts
//     finished runs in its high half (each run's workgroups add 2^32 in
//     total as they finish), and a run's epoch is one more than the count
//     it reads at launch, so no launch argument changes between runs;
//   * two sets of 8 tile-queue counters alternate by epoch parity: a run
//     uses one (zero when it starts) and its workgroup 0 zeroes the other,
//     which the next run takes;
//   * tile flags hold the epoch of the run that last published them, and a
//     consumer waits for (int32)(flag - epoch) >= 0;
//   * row counters grow by N1t per run; a consumer of run e waits for
//     (int32)(count - e * N1t) >= 0;
//   * split-K arrival counters are set back to zero by the last part of
//     each tile.
// So every policy's launches depend on nothing the host changes between
// runs, and may be captured in a HIP graph and replayed.  The epoch
// arithmetic is modular 32-bit, so wrap-around is harmless.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <string>

#include "../../include/mlp_chain.h"
#include "chain_launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

constexpr uint32_t DEFAULT_SPIN_LIMIT = 1u << 20;   // ~1 s of polling with back-off

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

uint32_t cdiv(int64_t a, int64_t b) { return (uint32_t)((a + b - 1) / b); }

}  // namespace

struct mlp_chain {
    int64_t M, H, I;
    int64_t ldt;                // row stride of T: I rounded up to 64 elements
    int64_t ldy;                // row stride of the kept layer outputs: H rounded up to 64 elements
    uint32_t layers;            // MLP layers of the chain (2 GEMMs each)
    int act, dtype, policy;
    int device;
    int cus;
    int cfg;
    int forced_cfg;
    int forced_s1, forced_s2;   // 0 = planner's split
    int forced_grid;            // 0 = planner's persistent grid
    int forced_order;           // -1 = planner's tile order
    int forced_rx;              // 0 = planner's XCD grid rows
    uint32_t order;             // bit 0 / 1: GEMM1 / GEMM2 tiles column-major in each XCD block
    CfgInfo ci;
    uint32_t Mt, N1t, N2t, T1, T2;
    uint32_t S1, S2, ksp1, ksp2;  // K split of GEMM1 / GEMM2 tiles
    int occ;        // persistent workgroups per CU
    uint32_t grid;  // persistent grid
    // workspace (one allocation, rebuilt when the plan changes)
    void* ws;
    size_t ws_bytes;
    size_t sync_bytes;          // the zeroed region: flags .. zero page
    uint16_t* t;
    uint16_t* ys;               // layers > 1: the outputs of every layer but the last
    uint32_t* flags;
    uint32_t* rowcnt;
    uint32_t* cnt1;
    uint32_t* cnt2;
    uint32_t* rdy1;
    uint32_t* rdy2;
    uint32_t* ticket;
    uint32_t* status;
    uint16_t* zero;
    uint64_t* run_epoch;        // high half: the last finished fused run's epoch
    float* part1;
    float* part2;
    // run state
    int64_t ldw1, ldw2;         // weight row strides (elements)
    uint32_t spin_limit;
    uint32_t skip_producer;
    uint64_t* trace;            // caller's timeline buffer (debug), or nullptr
    hipStream_t last_stream;
};

namespace {

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

constexpr int LDS_PER_CU = 160 * 1024;        // gfx950
constexpr size_t TICKET_BYTES = 2 * 8 * 256;  // two sets of 8 tile-queue counters, one per 256 bytes
constexpr uint32_t MIN_SLABS_PER_PART = 24;  // 1536 K-elements: keeps the partial traffic small
constexpr uint32_t MIN_SLABS_SHARED = 32;    // 2048 K-elements

// Deterministic split of each tile's K range when a GEMM has too few tiles
// to keep every CU busy.  (The CuSync README names CUTLASS StreamK as the
// other way to fill the last wave; this is a fixed split with a fixed-order
// reduction, so results stay bit-identical across policies.)  Targets,
// measured on the GPT-3, LLaMA-65 and Llama-2 shards over M = 1..2048 and
// every split up to 16:
//   * weight streaming (M < 256): about 3/4 of a part per CU when a single
//     row block reads each weight panel once, at most one part per CU
//     otherwise -- more parts add partial-sum traffic without adding
//     bandwidth;
//   * otherwise no split once the GEMM has a tile per CU (a workgroup alone
//     on a CU runs much faster than one of two), else as many parts as fit
//     one wave of the configuration's workgroups per CU (at most two).
// Every part keeps at least MIN_SLABS_PER_PART slabs (MIN_SLABS_SHARED when
// several row blocks read each weight panel): on the LLaMA-65 and Llama-2
// shards (K = 2752 and 3584 for GEMM2) shorter parts lost more to the fp32
// partial sums than the split gained.
// Tile order inside each XCD's block of the tile grid (bit 0: GEMM1, bit 1:
// GEMM2; set = column-major).  Does not change any output element.  Row-major
// for both GEMMs and every policy: on the GPT-3 shard, column-major GEMM2
// tiles cut the fused run's speed by 6% at M=2048 (an XCD's first consumers
// then need all of its row blocks, not just the first) and gained the
// stream-ordered pair at most 2% at M=2048 while losing 4% at M=1024.
uint32_t plan_order(int policy) {
    (void)policy;
    return 0u;
}

uint32_t plan_split(uint32_t tiles, uint32_t nks, int cus, int64_t M, uint32_t Mt, uint32_t wg_per_cu) {
    uint32_t s;
    if (Mt == 1) {
        s = (3u * (uint32_t)cus / 4u + tiles / 2) / tiles;
    } else if (M < 256) {
        s = (uint32_t)cus / tiles;
    } else if (tiles >= (uint32_t)cus) {
        s = 1;
    } else {
        s = (wg_per_cu < 2 ? wg_per_cu : 2u) * (uint32_t)cus / tiles;
    }
    const uint32_t cap = nks / (Mt == 1 ? MIN_SLABS_PER_PART : MIN_SLABS_SHARED);
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    const uint32_t ksp = (nks + s - 1) / s;      // no empty parts
    return (nks + ksp - 1) / ksp;
}

// Planner.  Tile configurations (chain_configs.h), chosen by M and tile
// counts; crossovers measured on the GPT-3, LLaMA-65, Llama-2 and 8192^3
// shards for M in 1..8192:
//   * M <= 16: 16 x 64 tiles, four LDS stages (weight streaming);
//   * M <= 256 while each GEMM has at most one 64 x 128 tile per CU: those
//     tiles with four stages and one workgroup per CU (three slabs of
//     weights in flight per CU);
//   * otherwise 256 x 128 tiles (eight waves of 64 x 64, three stages) or
//     256 x 256 tiles (eight waves of 128 x 64, a third fewer operand bytes
//     per MFMA; four stages of half a slab, which ran 2-6% faster than two
//     of a whole slab on the 256 x 256 shapes) once there are enough of those: for the
//     stream-ordered pair when GEMM2 has a wave of them, for the fused
//     policies when GEMM1 fills 7/8 of a wave (with fewer producer tiles the
//     consumers start early and wait);
//   * except where GEMM1 is split in two for the fused policies (below).
constexpr int CFG_SMALL = 0;    // 16 x 64, four stages
constexpr int CFG_DEEP = 4;     // 64 x 128, four stages, one workgroup per CU
constexpr int CFG_WIDE = 3;     // 256 x 128, eight waves, three stages
constexpr int CFG_BIG = 8;      // 256 x 256, eight waves of 128 x 64, four stages of half a slab

// Fused split of GEMM1.  When GEMM1's unsplit tiles make more than half a
// wave and at most one, every producer tile runs at once, all of them finish
// together, and the CUs without one idle until then (each consumer reads a
// whole row block of T).  Split in two, the producer parts make 1.5 waves of
// half-length items and the consumers of the first completed row blocks
// fill the last half wave: the stream-ordered pair's GEMM1 cannot do that
// (two rounds of half-length parts take as long as one of whole tiles).  It
// pays only when each part keeps at least MIN_SLABS_FUSED_SPLIT slabs, so
// that the fp32 partials and the reduction stay small against the K loop:
// on the GPT-3 shard (H = 12288, 96-slab parts) the fused run took 323 us
// instead of 370 at M = 1024 and 578 instead of 615 at M = 2048; on the
// LLaMA-65 and Llama-2 shards (H = 8192, 64-slab parts) it lost 5-15%.  The
// split is shared by every policy (bit-identical outputs), so the
// stream-ordered pair runs it too, in its own best configuration for it.
constexpr uint32_t MIN_SLABS_FUSED_SPLIT = 96;

struct Tiling {
    uint32_t mt, t1, t2;    // row blocks, GEMM1 tiles, GEMM2 tiles
    uint32_t wg;            // workgroups per CU the configuration's LDS ring allows
};

Tiling tiling(int64_t M, int64_t H, int64_t I, int act, int cfg) {
    const CfgInfo c = mlpc_config_info(cfg);
    const uint32_t mt = cdiv(M, c.BM);
    return {mt, mt * cdiv(I, act == MLP_ACT_SWIGLU ? c.BN / 2 : c.BN), mt * cdiv(H, c.BN),
            (uint32_t)(LDS_PER_CU / c.lds)};
}

// The configuration GEMM1 is split in two for (fused policies), or -1; its
// GEMM2 split in *s2.
int fused_split_config(int64_t M, int64_t H, int64_t I, int act, int cus, uint32_t* s2) {
    if (cdiv(H, mlpc::BK) < 2 * MIN_SLABS_FUSED_SPLIT) return -1;
    for (int cfg : {CFG_BIG, CFG_WIDE}) {
        const Tiling t = tiling(M, H, I, act, cfg);
        if (2 * t.t1 > (uint32_t)cus && t.t1 <= (uint32_t)cus) {
            *s2 = plan_split(t.t2, cdiv(I, mlpc::BK), cus, M, t.mt, t.wg);
            return cfg;
        }
    }
    return -1;
}

// Stream-ordered cost of a configuration under a given split: each kernel
// takes one round per wave of its tile parts, each round as long as one
// part's K slabs; a 256 x 128 slab step costs 0.625 of a 256 x 256 one
// (its MFMA rate per flop is 80%: more operand bytes per MFMA).  This wave
// rounding picked the faster configuration of the two in every measured
// stream-ordered case with a 2-way GEMM1 split.
double so_cost(int64_t M, int64_t H, int64_t I, int act, int cus, int cfg, uint32_t s1, uint32_t s2) {
    const Tiling t = tiling(M, H, I, act, cfg);
    const double slab = cfg == CFG_BIG ? 1.0 : 0.625;
    const uint32_t wave = (uint32_t)cus * t.wg;
    const uint32_t k1 = cdiv(cdiv(H, mlpc::BK), s1), k2 = cdiv(cdiv(I, mlpc::BK), s2);
    return slab * ((double)cdiv((int64_t)t.t1 * s1, wave) * k1 + (double)cdiv((int64_t)t.t2 * s2, wave) * k2);
}

// The small-M configuration, or -1 where the large tiles apply.  (64 x 128
// tiles need GEMM2 to have fewer tiles than CUs: on the LLaMA-65 shard at
// M = 256, exactly one wave of them, 256 x 128 tiles with K split 4 / 1 ran
// 4% faster fused.)
int small_config(int64_t M, int64_t H, int64_t I, int act, int cus) {
    if (M <= 16) return CFG_SMALL;
    if (M <= 256) {
        const Tiling t = tiling(M, H, I, act, CFG_DEEP);
        if (t.t1 <= (uint32_t)cus && t.t2 < (uint32_t)cus) return CFG_DEEP;
    }
    return -1;
}

// Measured plans of the benchmarked shapes (tuned_plans.inc, written by
// consumer_gemm_chain_amd/tune.py on the GPU): one K split per shape shared
// by every policy, and each policy's fastest tile configuration under it.
// A plan applies only to the exact sizes and CU count it was measured on;
// every other shape is planned by the rules below.
struct TunedPlan {
    int64_t M, H, I;
    int act, cus;
    uint32_t s1, s2;
    int cfg[3];   // per policy: stream_ordered, row_sync, tile_sync
};

const TunedPlan TUNED[] = {
#define MLPC_TUNED(m, h, i, act, cus, s1, s2, c0, c1, c2) {m, h, i, act, cus, s1, s2, {c0, c1, c2}},
#include "tuned_plans.inc"
#undef MLPC_TUNED
    {0, 0, 0, -1, 0, 1, 1, {-1, -1, -1}},   // end of the table
};

// While set on this thread, the planner ignores the tuned table (host-only
// plans of the rules, for tests).
thread_local bool g_rules_only = false;

struct RulesOnly {
    bool prev;
    explicit RulesOnly(bool on) : prev(g_rules_only) { g_rules_only = on; }
    ~RulesOnly() { g_rules_only = prev; }
};

const TunedPlan* tuned_plan(int64_t M, int64_t H, int64_t I, int act, int cus) {
    if (g_rules_only) return nullptr;
    for (const TunedPlan& t : TUNED)
        if (t.M == M && t.H == H && t.I == I && t.act == act && t.cus == cus) return &t;
    return nullptr;
}

int plan_config(int64_t M, int64_t H, int64_t I, int act, int policy, int cus) {
    if (const TunedPlan* tp = tuned_plan(M, H, I, act, cus)) return tp->cfg[policy];
    const int sc = small_config(M, H, I, act, cus);
    if (sc >= 0) return sc;
    uint32_t s2 = 1;
    const int fc = fused_split_config(M, H, I, act, cus, &s2);
    if (fc >= 0) {
        if (policy != MLP_POLICY_STREAM_ORDERED) return fc;
        return so_cost(M, H, I, act, cus, CFG_BIG, 2, s2) <= so_cost(M, H, I, act, cus, CFG_WIDE, 2, s2)
                   ? CFG_BIG : CFG_WIDE;
    }
    const Tiling t = tiling(M, H, I, act, CFG_BIG);
    if (policy == MLP_POLICY_STREAM_ORDERED ? t.t2 >= (uint32_t)cus : 8 * t.t1 >= 7 * (uint32_t)cus)
        return CFG_BIG;
    return CFG_WIDE;
}

// The K split every policy uses for (M, H, I, act): the fused split of
// GEMM1 where it applies, else the split rule above on the tiling of the
// stream-ordered plan.
void plan_shared_split(int64_t M, int64_t H, int64_t I, int act, int cus, uint32_t* s1, uint32_t* s2) {
    if (const TunedPlan* tp = tuned_plan(M, H, I, act, cus)) {
        *s1 = tp->s1;
        *s2 = tp->s2;
        return;
    }
    if (small_config(M, H, I, act, cus) < 0 && fused_split_config(M, H, I, act, cus, s2) >= 0) {
        *s1 = 2;
        return;
    }
    const Tiling t = tiling(M, H, I, act, plan_config(M, H, I, act, MLP_POLICY_STREAM_ORDERED, cus));
    *s1 = plan_split(t.t1, cdiv(H, mlpc::BK), cus, M, t.mt, t.wg);
    *s2 = plan_split(t.t2, cdiv(I, mlpc::BK), cus, M, t.mt, t.wg);
}

// The tiling and K split of configuration `cfg` for (M, H, I, act) on `cus`
// CUs; forced splits (> 0) replace the planned ones.
struct TilePlan {
    CfgInfo ci;
    uint32_t Mt, N1t, N2t, T1, T2;
    uint32_t S1, S2, ksp1, ksp2;
};

TilePlan tile_plan(int64_t M, int64_t H, int64_t I, int act, int cus, int cfg, int forced_s1, int forced_s2) {
    TilePlan p{};
    p.ci = mlpc_config_info(cfg);
    p.Mt = cdiv(M, p.ci.BM);
    p.N1t = cdiv(I, act == MLP_ACT_SWIGLU ? p.ci.BN / 2 : p.ci.BN);
    p.N2t = cdiv(H, p.ci.BN);
    p.T1 = p.Mt * p.N1t;
    p.T2 = p.Mt * p.N2t;
    // The split does not depend on the policy or on `cfg`, so every policy
    // splits K alike.  The tile shape does not change any output element's
    // arithmetic (same MFMA sequence over the same slabs), the split does:
    // equal splits keep the policies bit-identical while each uses its own
    // tile configuration.
    uint32_t s1 = 1, s2 = 1;
    plan_shared_split(M, H, I, act, cus, &s1, &s2);
    p.S1 = forced_s1 > 0 ? (uint32_t)forced_s1 : s1;
    p.S2 = forced_s2 > 0 ? (uint32_t)forced_s2 : s2;
    const uint32_t nks1 = cdiv(H, mlpc::BK), nks2 = cdiv(I, mlpc::BK);
    p.ksp1 = (nks1 + p.S1 - 1) / p.S1;
    p.ksp2 = (nks2 + p.S2 - 1) / p.S2;
    return p;
}

// (Re)compute the tiling of a handle for configuration `cfg` and the splits.
int apply_plan(mlp_chain* h, int cfg) {
    if (mlpc_config_info(cfg).id < 0) return fail(MLP_EINVAL, "unknown tile configuration %d", cfg);
    const TilePlan p = tile_plan(h->M, h->H, h->I, h->act, h->cus, cfg, h->forced_s1, h->forced_s2);
    h->cfg = cfg;
    h->ci = p.ci;
    h->Mt = p.Mt;
    h->N1t = p.N1t;
    h->N2t = p.N2t;
    h->T1 = p.T1;
    h->T2 = p.T2;
    h->S1 = p.S1;
    h->S2 = p.S2;
    h->ksp1 = p.ksp1;
    h->ksp2 = p.ksp2;
    h->order = h->forced_order >= 0 ? (uint32_t)h->forced_order : plan_order(h->policy);
    h->occ = 0;
    h->grid = 0;
    if (h->policy != MLP_POLICY_STREAM_ORDERED) {
        int occ = 0;
        hipError_t e = mlpc_persistent_occupancy(cfg, h->dtype, h->policy, (int)h->layers, &occ);
        if (e != hipSuccess) return fail(MLP_EHIP, "occupancy query failed: %s", hipGetErrorString(e));
        if (occ < 1) return fail(MLP_EHIP, "persistent kernel of config %d does not fit on a CU", cfg);
        h->occ = occ;
        // Persistent workgroups: as many per CU as fit, but no more than the
        // whole items per CU one layer has (the layers of a chain run one
        // after another, so one layer's parts are what can run at once; extra
        // workgroups would only sit on the next layer's items and wait).
        // When a layer is under two items per CU (small M), one workgroup per
        // CU runs a producer part and then a consumer part, so the consumers
        // spread over the CUs the producers used instead of sharing the CUs
        // their workgroups were placed on at launch.
        const uint64_t layer_parts = (uint64_t)h->T1 * h->S1 + (uint64_t)h->T2 * h->S2;
        uint64_t per_cu = layer_parts / (uint64_t)h->cus;
        if (per_cu < 1) per_cu = 1;
        if (per_cu > (uint64_t)occ) per_cu = (uint64_t)occ;
        uint64_t g = per_cu * (uint64_t)h->cus;
        if (g > layer_parts * h->layers) g = layer_parts * h->layers;
        // at least one workgroup per tile queue (the kernel's deadlock-freedom
        // argument needs an owner for every queue); extras exit at once
        if (g < 8) g = 8;
        if (h->forced_grid > 0) {
            g = (uint64_t)h->forced_grid;
            if (g > (uint64_t)occ * (uint64_t)h->cus) g = (uint64_t)occ * (uint64_t)h->cus;
            if (g < 8) g = 8;
        }
        h->grid = (uint32_t)g;
    }
    return MLP_OK;
}

int zero_workspace(mlp_chain* h) {
    hipError_t e = hipMemset(h->flags, 0, h->sync_bytes);
    if (e != hipSuccess) return fail(MLP_EHIP, "hipMemset failed: %s", hipGetErrorString(e));
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(MLP_EHIP, "hipDeviceSynchronize failed: %s", hipGetErrorString(e));
    return MLP_OK;
}

// Words between the 8 copies of the ready flags, one per XCD: the flags of
// all layers, rounded up to 1 KB, plus 128 bytes, so that each copy starts
// on the next class of 128-byte lines (another memory channel).  Producers
// publish into every copy; the consumers of an XCD poll their own copy, so
// the hundreds of consumers that may wait at small M spread their polls over
// eight sets of lines instead of one.
uint32_t flag_stride(const mlp_chain* h) {
    const size_t n = (size_t)h->layers * h->T1 + (size_t)(h->layers - 1) * h->T2;
    return (uint32_t)(align_up(n, 256) + 32);
}

// Workspace layout of the current plan at `base` (nullptr: sizes only), for
// a chain of L = layers MLP layers:
//   T [L][M, ldt] | Y [L-1][M, ldy] | flags [8][fstride >= L T1 + (L-1) T2] | rowcnt [(2L-1) Mt] | cnt1 [L T1] |
//   cnt2 [L T2] | rdy1 [L T1 S1] | rdy2 [L T2 S2] | ticket | status | zero page | part1 [L] | part2 [L]
// (flags .. zero page, sync_bytes long, is the region that starts at zero).
// Sets ws_bytes and sync_bytes; with a base also every buffer pointer.
void layout_workspace(mlp_chain* h, char* base) {
    const size_t L = h->layers;
    const size_t acc_bytes = (size_t)h->ci.BM * h->ci.BN * 4;     // one tile's fp32 accumulators
    const size_t t_b = align_up(L * (size_t)h->M * (size_t)h->ldt * 2, 256);
    const size_t ys_b = align_up((L - 1) * (size_t)h->M * (size_t)h->ldy * 2, 256);
    const size_t f_b = align_up(8 * (size_t)flag_stride(h) * 4, 256);
    const size_t r_b = align_up((2 * L - 1) * h->Mt * 4, 256);
    const size_t c1_b = align_up(L * h->T1 * 4, 256);
    const size_t c2_b = align_up(L * h->T2 * 4, 256);
    const size_t p1_b = h->S1 > 1 ? align_up(L * h->T1 * h->S1 * acc_bytes, 256) : 0;
    const size_t p2_b = h->S2 > 1 ? align_up(L * h->T2 * h->S2 * acc_bytes, 256) : 0;
    const size_t y1_b = align_up(L * h->T1 * h->S1 * 4, 256);
    const size_t y2_b = align_up(L * h->T2 * h->S2 * 4, 256);
    h->sync_bytes = f_b + r_b + c1_b + c2_b + y1_b + y2_b + TICKET_BYTES + 3 * 256;
    h->ws_bytes = t_b + ys_b + h->sync_bytes + p1_b + p2_b;
    if (!base) return;
    char* p = base;
    h->t = reinterpret_cast<uint16_t*>(p);
    p += t_b;
    h->ys = ys_b ? reinterpret_cast<uint16_t*>(p) : nullptr;
    p += ys_b;
    h->flags = reinterpret_cast<uint32_t*>(p);
    p += f_b;
    h->rowcnt = reinterpret_cast<uint32_t*>(p);
    p += r_b;
    h->cnt1 = reinterpret_cast<uint32_t*>(p);
    p += c1_b;
    h->cnt2 = reinterpret_cast<uint32_t*>(p);
    p += c2_b;
    h->rdy1 = reinterpret_cast<uint32_t*>(p);
    p += y1_b;
    h->rdy2 = reinterpret_cast<uint32_t*>(p);
    p += y2_b;
    h->ticket = reinterpret_cast<uint32_t*>(p);            // 2 sets of 8 queue counters, 256 B apart
    h->status = reinterpret_cast<uint32_t*>(p + TICKET_BYTES);
    h->zero = reinterpret_cast<uint16_t*>(p + TICKET_BYTES + 256);
    h->run_epoch = reinterpret_cast<uint64_t*>(p + TICKET_BYTES + 2 * 256);
    p += TICKET_BYTES + 3 * 256;
    h->part1 = p1_b ? reinterpret_cast<float*>(p) : nullptr;
    p += p1_b;
    h->part2 = p2_b ? reinterpret_cast<float*>(p) : nullptr;
}

// Allocate (or re-allocate) and zero the workspace for the current plan.
int build_workspace(mlp_chain* h) {
    if (h->ws) {
        (void)hipDeviceSynchronize();
        (void)hipFree(h->ws);
        h->ws = nullptr;
    }
    layout_workspace(h, nullptr);
    hipError_t e = hipMalloc(&h->ws, h->ws_bytes);
    if (e != hipSuccess) {
        h->ws = nullptr;
        return fail(MLP_ENOMEM, "hipMalloc of %zu workspace bytes failed: %s", h->ws_bytes, hipGetErrorString(e));
    }
    layout_workspace(h, static_cast<char*>(h->ws));
    return zero_workspace(h);
}

bool bad_ptr(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) != 0; }

mlpc::ChainArgs make_args(const mlp_chain* h, const void* x, const void* w1, const void* w2, void* out) {
    mlpc::ChainArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.w1 = static_cast<const uint16_t*>(w1);
    a.w2 = static_cast<const uint16_t*>(w2);
    a.t = h->t;
    a.y = static_cast<uint16_t*>(out);
    a.M = (int)h->M;
    a.H = (int)h->H;
    a.I = (int)h->I;
    a.ldt = (int)h->ldt;
    a.act = h->act;
    // producer tiles narrower than 64 columns share 128-byte lines of T
    a.acq_agent = ((h->act == MLP_ACT_SWIGLU ? h->ci.BN / 2 : h->ci.BN) % 64) != 0 ? 1u : 0u;
    a.Mt = h->Mt;
    a.N1t = h->N1t;
    a.N2t = h->N2t;
    a.T1 = h->T1;
    a.T2 = h->T2;
    a.rx = h->forced_rx > 0 ? (uint32_t)h->forced_rx : h->Mt >= 2 ? 2u : 1u;
    a.order = h->order;
    a.ticket = h->ticket;
    a.run_epoch = h->run_epoch;
    a.flags = h->flags;
    a.fstride = flag_stride(h);
    a.rowcnt = h->rowcnt;
    a.status = h->status;
    a.zero = h->zero;
    a.S1 = h->S1;
    a.S2 = h->S2;
    a.ksp1 = h->ksp1;
    a.ksp2 = h->ksp2;
    a.part1 = h->part1;
    a.part2 = h->part2;
    a.cnt1 = h->cnt1;
    a.cnt2 = h->cnt2;
    a.rdy1 = h->rdy1;
    a.rdy2 = h->rdy2;
    a.grid = h->grid;
    a.spin_limit = h->spin_limit;
    a.skip_producer = h->skip_producer;
    a.trace = h->trace;
    a.ldx = (int)h->H;
    a.ldo = (int)h->H;
    a.ldw1 = (int)h->ldw1;
    a.ldw2 = (int)h->ldw2;
    a.layers = h->layers;
    a.ldy = (int)h->ldy;
    a.ys = h->ys;
    a.w1s[0] = a.w1;
    a.w2s[0] = a.w2;
    a.policy = h->policy;
    return a;
}

// The handle's sizes and defaults (no plan, no workspace yet).
void init_handle(mlp_chain* h, int64_t M, int64_t H, int64_t I, int act, int dtype, int policy, int dev, int cus,
                 int layers = 1) {
    h->M = M;
    h->H = H;
    h->I = I;
    h->ldt = (I + 63) / 64 * 64;
    h->ldy = (H + 63) / 64 * 64;
    h->ldw1 = (act == MLP_ACT_SWIGLU ? 2 : 1) * I;
    h->ldw2 = H;
    h->layers = (uint32_t)layers;
    h->ys = nullptr;
    h->act = act;
    h->dtype = dtype;
    h->policy = policy;
    h->device = dev;
    h->cus = cus;
    h->forced_cfg = -1;
    h->forced_s1 = 0;
    h->forced_grid = 0;
    h->forced_order = -1;
    h->forced_rx = 0;
    h->forced_s2 = 0;
    h->spin_limit = DEFAULT_SPIN_LIMIT;
    h->skip_producer = mlpc::NO_SKIP;
    h->trace = nullptr;
    h->last_stream = nullptr;
    h->ws = nullptr;
}

// Argument checks shared by create and plan.
int check_chain_args(int64_t M, int64_t H, int64_t I, int act, int policy) {
    if (M < 1 || H < 8 || I < 8)
        return fail(MLP_EINVAL, "sizes must be M >= 1, H >= 8, I >= 8 (got M=%lld H=%lld I=%lld)",
                    (long long)M, (long long)H, (long long)I);
    if (H % 8 != 0 || I % 8 != 0)
        return fail(MLP_EINVAL, "H and I must be multiples of 8 (16-byte rows), got H=%lld I=%lld",
                    (long long)H, (long long)I);
    // Every operand stays below 2^31 bytes and every row below 2^23 elements
    // (32-bit element and byte offsets within an operand cannot wrap).
    const int64_t lim = (int64_t)1 << 30;
    if (M * H >= lim || M * I >= lim || H * I * 2 >= lim || M >= (1 << 24) || H > (1 << 22) || I > (1 << 22))
        return fail(MLP_EINVAL, "sizes too large for 32-bit tile indexing (M=%lld H=%lld I=%lld)",
                    (long long)M, (long long)H, (long long)I);
    if (act < MLP_ACT_NONE || act > MLP_ACT_SWIGLU) return fail(MLP_EINVAL, "unknown activation %d", act);
    if (policy < MLP_POLICY_STREAM_ORDERED || policy > MLP_POLICY_TILE_SYNC)
        return fail(MLP_EINVAL, "unknown policy %d", policy);
    return MLP_OK;
}

}  // namespace

extern "C" {

const char* mlp_chain_last_error(void) { return g_err.c_str(); }

mlp_chain_t mlp_chain_create(int64_t M, int64_t H, int64_t I, int act, int dtype, int policy) {
    return mlp_chain_create_layers(M, H, I, act, dtype, policy, 1);
}

mlp_chain_t mlp_chain_create_layers(int64_t M, int64_t H, int64_t I, int act, int dtype, int policy, int layers) {
    g_err.clear();
    if (check_chain_args(M, H, I, act, policy) != MLP_OK) return nullptr;
    if (layers < 1 || layers > (int)mlpc::MAX_LAYERS) {
        fail(MLP_EINVAL, "layers must be in 1..%u, got %d", mlpc::MAX_LAYERS, layers);
        return nullptr;
    }
    if (dtype != MLP_DTYPE_F16 && dtype != MLP_DTYPE_BF16) {
        fail(MLP_EINVAL, "unknown dtype %d", dtype);
        return nullptr;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        fail(MLP_EHIP, "no HIP device: %s", hipGetErrorString(e));
        return nullptr;
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
        fail(MLP_EHIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
        return nullptr;
    }
    mlp_chain* h = new (std::nothrow) mlp_chain();
    if (!h) {
        fail(MLP_ENOMEM, "out of host memory");
        return nullptr;
    }
    init_handle(h, M, H, I, act, dtype, policy, dev, prop.multiProcessorCount, layers);
    if (apply_plan(h, plan_config(M, H, I, act, policy, h->cus)) != MLP_OK || build_workspace(h) != MLP_OK) {
        if (h->ws) (void)hipFree(h->ws);
        delete h;
        return nullptr;
    }
    return h;
}

int mlp_chain_destroy(mlp_chain_t h) {
    if (!h) return MLP_OK;
    DeviceGuard g(h->device);
    // the handle's work is ordered on the stream of its last run
    hipError_t e1 = hipStreamSynchronize(h->last_stream);
    hipError_t e2 = hipFree(h->ws);
    delete h;
    if (e1 != hipSuccess || e2 != hipSuccess)
        return fail(MLP_EHIP, "destroy: %s", hipGetErrorString(e1 != hipSuccess ? e1 : e2));
    return MLP_OK;
}

static int launch_phase(mlp_chain_t h, int what, const mlpc::ChainArgs& a, hipStream_t s) {
    hipError_t e = mlpc_launch(a, h->cfg, h->dtype, what, (int)h->grid, s);
    if (e != hipSuccess) return fail(MLP_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return MLP_OK;
}

int mlp_chain_run_layers(mlp_chain_t h, const void* x, const void* const* w1, const void* const* w2, void* out,
                         void* hip_stream) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    if (!w1 || !w2) return fail(MLP_EINVAL, "w1 and w2 must be host arrays of the layers' weight pointers");
    for (uint32_t l = 0; l < h->layers; ++l)
        if (bad_ptr(w1[l]) || bad_ptr(w2[l]))
            return fail(MLP_EINVAL, "layer %u: w1 and w2 must be non-NULL 16-byte aligned device pointers", l);
    if (bad_ptr(x) || bad_ptr(out))
        return fail(MLP_EINVAL, "x and out must be non-NULL 16-byte aligned device pointers");
    if (h->layers == 1) return mlp_chain_run(h, x, w1[0], w2[0], out, hip_stream);
    DeviceGuard g(h->device);
    if (!g.ok) return fail(MLP_EHIP, "cannot select the handle's device %d", h->device);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    h->last_stream = s;
    const bool fused = h->policy != MLP_POLICY_STREAM_ORDERED;
    mlpc::ChainArgs a = make_args(h, x, w1[0], w2[0], out);
    for (uint32_t l = 0; l < h->layers; ++l) {
        a.w1s[l] = static_cast<const uint16_t*>(w1[l]);
        a.w2s[l] = static_cast<const uint16_t*>(w2[l]);
    }
    if (!fused) {
        // 2 x layers kernels on the stream, layer by layer
        for (uint32_t l = 0; l < h->layers; ++l) {
            const mlpc::ChainArgs b = mlpc::layer_args(a, l, (size_t)h->ci.BM * h->ci.BN);
            int rc = launch_phase(h, LAUNCH_GEMM1, b, s);
            if (rc == MLP_OK) rc = launch_phase(h, LAUNCH_GEMM2, b, s);
            if (rc != MLP_OK) return rc;
        }
        return MLP_OK;
    }
    return launch_phase(h, h->policy == MLP_POLICY_ROW_SYNC ? LAUNCH_LAYERS_ROW : LAUNCH_LAYERS_TILE, a, s);
}

int mlp_chain_run(mlp_chain_t h, const void* x, const void* w1, const void* w2, void* out, void* hip_stream) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    if (h->layers != 1)
        return fail(MLP_EINVAL, "the handle chains %u layers: run it with mlp_chain_run_layers", h->layers);
    if (bad_ptr(x) || bad_ptr(w1) || bad_ptr(w2) || bad_ptr(out))
        return fail(MLP_EINVAL, "x, w1, w2 and out must be non-NULL 16-byte aligned device pointers");
    DeviceGuard g(h->device);
    if (!g.ok) return fail(MLP_EHIP, "cannot select the handle's device %d", h->device);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    h->last_stream = s;
    if (h->policy == MLP_POLICY_STREAM_ORDERED) {
        const mlpc::ChainArgs a = make_args(h, x, w1, w2, out);
        int rc = launch_phase(h, LAUNCH_GEMM1, a, s);
        if (rc == MLP_OK) rc = launch_phase(h, LAUNCH_GEMM2, a, s);
        return rc;   // (a failed launch leaves the device unusable; counters need not roll back)
    }
    // the run's epoch is the device's (one more than the last finished
    // run's), so nothing here changes between runs and the launch may be
    // captured into a graph
    const mlpc::ChainArgs a = make_args(h, x, w1, w2, out);
    return launch_phase(h, h->policy == MLP_POLICY_ROW_SYNC ? LAUNCH_ROW : LAUNCH_TILE, a, s);
}

int mlp_chain_run_noalloc(int64_t M, int64_t H, int64_t I, int act, int dtype, int policy, const void* x,
                          const void* w1, const void* w2, void* out, void* status, void* hip_stream) {
    if (check_chain_args(M, H, I, act, policy) != MLP_OK) return MLP_EINVAL;
    if (dtype != MLP_DTYPE_F16 && dtype != MLP_DTYPE_BF16) return fail(MLP_EINVAL, "unknown dtype %d", dtype);
    if (bad_ptr(x) || bad_ptr(w1) || bad_ptr(w2) || bad_ptr(out))
        return fail(MLP_EINVAL, "x, w1, w2 and out must be non-NULL 16-byte aligned device pointers");
    if (((uintptr_t)status & 3u) != 0) return fail(MLP_EINVAL, "status must be a 4-byte aligned device pointer or NULL");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(MLP_EHIP, "no HIP device: %s", hipGetErrorString(e));
    void* base = nullptr;
    e = mlpc_scratch_address(dev, &base);
    if (e != hipSuccess) return fail(MLP_EHIP, "device %d: scratch address lookup failed: %s", dev, hipGetErrorString(e));
    // A handle on the stack: the same plan mlp_chain_create makes, with its
    // workspace laid out in the static scratch instead of an allocation.
    mlp_chain h{};
    init_handle(&h, M, H, I, act, dtype, policy, dev, cus);
    const int rc = apply_plan(&h, plan_config(M, H, I, act, policy, cus));
    if (rc != MLP_OK) return rc;
    layout_workspace(&h, nullptr);
    if (h.ws_bytes > MLPC_SCRATCH_BYTES)
        return fail(MLP_EINVAL, "M=%lld H=%lld I=%lld needs %zu bytes of workspace; the static scratch holds %zu "
                    "(use mlp_chain_create / mlp_chain_run)", (long long)M, (long long)H, (long long)I,
                    h.ws_bytes, (size_t)MLPC_SCRATCH_BYTES);
    layout_workspace(&h, static_cast<char*>(base));
    if (status) h.status = static_cast<uint32_t*>(status);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    // Every call starts from zeroed synchronization words (flags, counters,
    // ready words, queue counters, status, zero page, epoch words: the run
    // is epoch 1), whatever an earlier call on this device left there.
    e = mlpc_zero_words(h.flags, h.sync_bytes, h.status, s);
    if (e != hipSuccess) return fail(MLP_EHIP, "clearing the scratch failed: %s", hipGetErrorString(e));
    const mlpc::ChainArgs a = make_args(&h, x, w1, w2, out);
    if (policy == MLP_POLICY_STREAM_ORDERED) {
        int r = launch_phase(&h, LAUNCH_GEMM1, a, s);
        if (r == MLP_OK) r = launch_phase(&h, LAUNCH_GEMM2, a, s);
        return r;
    }
    return launch_phase(&h, policy == MLP_POLICY_ROW_SYNC ? LAUNCH_ROW : LAUNCH_TILE, a, s);
}

int mlp_chain_run_phase(mlp_chain_t h, int phase, const void* x, const void* w1, const void* w2, void* out,
                        void* hip_stream) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    if (phase != 1 && phase != 2) return fail(MLP_EINVAL, "phase must be 1 or 2, got %d", phase);
    if (phase == 1 && (bad_ptr(x) || bad_ptr(w1)))
        return fail(MLP_EINVAL, "phase 1 needs non-NULL 16-byte aligned x and w1");
    if (phase == 2 && (bad_ptr(w2) || bad_ptr(out)))
        return fail(MLP_EINVAL, "phase 2 needs non-NULL 16-byte aligned w2 and out");
    DeviceGuard g(h->device);
    if (!g.ok) return fail(MLP_EHIP, "cannot select the handle's device %d", h->device);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    h->last_stream = s;
    const mlpc::ChainArgs a = make_args(h, x, w1, w2, out);
    return launch_phase(h, phase == 1 ? LAUNCH_GEMM1 : LAUNCH_GEMM2, a, s);
}

int mlp_chain_status(mlp_chain_t h) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    DeviceGuard g(h->device);
    // the status word is read on the stream of the handle's last run, after
    // that run: other streams of the process are not waited for
    uint32_t st = 0;
    hipError_t e = hipMemcpyAsync(&st, h->status, sizeof st, hipMemcpyDeviceToHost, h->last_stream);
    if (e == hipSuccess) e = hipStreamSynchronize(h->last_stream);
    if (e != hipSuccess) return fail(MLP_EHIP, "reading status failed: %s", hipGetErrorString(e));
    if (st != 0) {
        int rc = zero_workspace(h);
        if (rc != MLP_OK) return rc;
        return fail(MLP_ETIMEOUT, "a consumer tile gave up waiting for its producer (watchdog)");
    }
    return MLP_OK;
}

int mlp_chain_weight_ld(int64_t H, int64_t I, int act, int64_t* ldw1, int64_t* ldw2) {
    if (!ldw1 || !ldw2) return fail(MLP_EINVAL, "mlp_chain_weight_ld needs two output slots");
    if (H < 8 || I < 8 || H % 8 || I % 8 || act < MLP_ACT_NONE || act > MLP_ACT_SWIGLU)
        return fail(MLP_EINVAL, "bad sizes H=%lld I=%lld or act %d", (long long)H, (long long)I, act);
    // the next stride that is an odd number of 128-byte lines (64 mod 128
    // elements): consecutive rows of a column panel then cycle through all
    // eight classes of lines ((address / 128) mod 8)
    auto odd_lines = [](int64_t n) { return n + ((64 - n % 128) + 128) % 128; };
    *ldw1 = odd_lines((act == MLP_ACT_SWIGLU ? 2 : 1) * I);
    *ldw2 = odd_lines(H);
    return MLP_OK;
}

int mlp_chain_set_weight_ld(mlp_chain_t h, int64_t ldw1, int64_t ldw2) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    const int64_t g = h->act == MLP_ACT_SWIGLU ? 2 : 1;
    if (ldw1 < g * h->I || ldw2 < h->H || ldw1 % 8 || ldw2 % 8 || ldw1 > (1 << 24) || ldw2 > (1 << 24))
        return fail(MLP_EINVAL, "weight row strides must be multiples of 8 elements, ldw1 >= %lld, ldw2 >= %lld "
                    "and at most 2^24 (got %lld, %lld)", (long long)(g * h->I), (long long)h->H, (long long)ldw1,
                    (long long)ldw2);
    h->ldw1 = ldw1;
    h->ldw2 = ldw2;
    return MLP_OK;
}

int mlp_chain_info(mlp_chain_t h, int64_t* info, int n) {
    if (!h || !info || n < 16) return fail(MLP_EINVAL, "mlp_chain_info needs a handle and 16 slots");
    // the epoch of the last finished fused run, read on the stream of the
    // handle's last run, after it
    DeviceGuard g(h->device);
    uint64_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, h->run_epoch, sizeof word, hipMemcpyDeviceToHost, h->last_stream);
    if (e == hipSuccess) e = hipStreamSynchronize(h->last_stream);
    if (e != hipSuccess) return fail(MLP_EHIP, "reading the epoch failed: %s", hipGetErrorString(e));
    const uint32_t epoch = (uint32_t)(word >> 32);
    const int64_t bn1 = h->act == MLP_ACT_SWIGLU ? h->ci.BN / 2 : h->ci.BN;
    const int64_t v[21] = {h->ci.BM, bn1, h->ci.BN, h->ci.BK, h->Mt, h->N1t, h->N2t, h->T1, h->T2,
                           h->grid, h->occ, h->ci.NT, h->cus, epoch, h->cfg, (int64_t)h->ws_bytes,
                           h->S1, h->S2, h->ksp1, h->ksp2, h->layers};
    for (int i = 0; i < n && i < 21; ++i) info[i] = v[i];
    return MLP_OK;
}

int mlp_chain_debug_set_spin_limit(mlp_chain_t h, uint32_t limit) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    h->spin_limit = limit ? limit : DEFAULT_SPIN_LIMIT;
    return MLP_OK;
}

int mlp_chain_plan(int64_t M, int64_t H, int64_t I, int act, int policy, int cus, int64_t* plan, int n) {
    if (!plan || n < 3) return fail(MLP_EINVAL, "mlp_chain_plan needs an array of at least 3 slots");
    // cus < 0: the rules alone for -cus CUs (no tuned plan)
    const bool rules_only = cus < 0;
    if (rules_only) cus = -cus;
    if (cus < 8) return fail(MLP_EINVAL, "cus must be >= 8 (or <= -8), got %d", rules_only ? -cus : cus);
    RulesOnly scope(rules_only);
    const int rc = check_chain_args(M, H, I, act, policy);
    if (rc != MLP_OK) return rc;
    const int cfg = plan_config(M, H, I, act, policy, cus);
    const TilePlan p = tile_plan(M, H, I, act, cus, cfg, 0, 0);
    const int64_t bn1 = act == MLP_ACT_SWIGLU ? p.ci.BN / 2 : p.ci.BN;
    const int64_t v[14] = {cfg, p.S1, p.S2, p.ci.BM, bn1, p.ci.BN, p.Mt, p.N1t, p.N2t, p.T1, p.T2, p.ksp1, p.ksp2,
                           tuned_plan(M, H, I, act, cus) ? 1 : 0};
    for (int i = 0; i < n && i < 14; ++i) plan[i] = v[i];
    return MLP_OK;
}

int mlp_chain_debug_skip_producer(mlp_chain_t h, int64_t tile) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    const int64_t parts = (int64_t)h->T1 * h->S1;
    h->skip_producer = (tile < 0 || tile >= parts) ? mlpc::NO_SKIP : (uint32_t)tile;
    return MLP_OK;
}

static int replan(mlp_chain_t h) {
    DeviceGuard g(h->device);
    const int cfg = h->forced_cfg < 0 ? plan_config(h->M, h->H, h->I, h->act, h->policy, h->cus) : h->forced_cfg;
    int rc = apply_plan(h, cfg);
    if (rc != MLP_OK) return rc;
    return build_workspace(h);
}

int mlp_chain_debug_set_config(mlp_chain_t h, int config_id) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    if (config_id < -1 || config_id >= mlpc_num_configs())
        return fail(MLP_EINVAL, "unknown tile configuration %d", config_id);
    h->forced_cfg = config_id;
    return replan(h);
}

int mlp_chain_debug_set_grid(mlp_chain_t h, int grid) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    if (grid < 0) return fail(MLP_EINVAL, "grid must be >= 0, got %d", grid);
    h->forced_grid = grid;
    return apply_plan(h, h->cfg);
}

int mlp_chain_debug_set_order(mlp_chain_t h, int order) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    const int rx = order < 0 ? 0 : order >> 4;
    if (order < -1 || (order >= 0 && ((order & ~0xf3) != 0 || (rx != 0 && rx != 1 && rx != 2 && rx != 4 && rx != 8))))
        return fail(MLP_EINVAL, "order must be -1 (planned) or (0..3) | rx << 4 with rx in {0, 1, 2, 4, 8}, got %d",
                    order);
    h->forced_order = order < 0 ? -1 : order & 3;
    h->forced_rx = rx;
    return apply_plan(h, h->cfg);
}

int mlp_chain_debug_set_split(mlp_chain_t h, int s1, int s2) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    if (s1 < 0 || s2 < 0 || s1 > 64 || s2 > 64) return fail(MLP_EINVAL, "splits must be in 0..64");
    h->forced_s1 = s1;
    h->forced_s2 = s2;
    return replan(h);
}

int mlp_chain_debug_litmus(void* data, size_t data_bytes, void* flags, size_t flag_bytes, void* result, int rounds,
                           int half_lines, int agent, uint32_t spin_limit, void* hip_stream) {
    if (!data || !flags || !result || ((uintptr_t)data & 255u) != 0 || ((uintptr_t)flags & 3u) != 0 ||
        ((uintptr_t)result & 3u) != 0)
        return fail(MLP_EINVAL, "litmus: data (256-byte aligned), flags and result must be device pointers");
    if (rounds < 1 || rounds > 4096 || data_bytes < (size_t)rounds * (1u << 20) || flag_bytes < (size_t)rounds * 1024)
        return fail(MLP_EINVAL, "litmus: %d rounds need %zu data bytes and %zu flag bytes", rounds,
                    (size_t)rounds << 20, (size_t)rounds * 1024);
    const hipError_t e = mlpc_litmus(data, data_bytes, flags, flag_bytes, result, rounds, half_lines, agent,
                                     spin_limit ? spin_limit : DEFAULT_SPIN_LIMIT,
                                     static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(MLP_EHIP, "litmus launch failed: %s", hipGetErrorString(e));
    return MLP_OK;
}

int mlp_chain_debug_set_epoch(mlp_chain_t h, uint32_t epoch) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    DeviceGuard g(h->device);
    // flags and row counters as the run of epoch `epoch` leaves them: every
    // flag published with it, every row counter at epoch x tiles per row
    const uint32_t L = h->layers;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemsetD32(h->flags, (int)epoch, 8 * (size_t)flag_stride(h));
    if (e == hipSuccess) e = hipMemsetD32(h->rowcnt, (int)(epoch * h->N1t), L * h->Mt);
    if (e == hipSuccess && L > 1) e = hipMemsetD32(h->rowcnt + L * h->Mt, (int)(epoch * h->N2t), (L - 1) * h->Mt);
    // both sets of queue counters zero, the run count `epoch`
    const uint64_t word = (uint64_t)epoch << 32;
    if (e == hipSuccess) e = hipMemset(h->ticket, 0, TICKET_BYTES);
    if (e == hipSuccess) e = hipMemcpy(h->run_epoch, &word, sizeof word, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(MLP_EHIP, "setting the epoch failed: %s", hipGetErrorString(e));
    return MLP_OK;
}

int mlp_chain_debug_set_trace(mlp_chain_t h, void* buffer) {
    if (!h) return fail(MLP_EINVAL, "NULL handle");
    h->trace = static_cast<uint64_t*>(buffer);
    return MLP_OK;
}

int mlp_chain_debug_read_intermediate(mlp_chain_t h, void* dst, void* hip_stream) {
    if (!h || !dst) return fail(MLP_EINVAL, "mlp_chain_debug_read_intermediate needs a handle and a buffer");
    DeviceGuard g(h->device);
    hipError_t e = hipMemcpy2DAsync(dst, (size_t)h->I * 2, h->t, (size_t)h->ldt * 2, (size_t)h->I * 2,
                                    (size_t)h->M, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(MLP_EHIP, "copy of the intermediate failed: %s", hipGetErrorString(e));
    return MLP_OK;
}

}  // extern "C"
