// chain_litmus.hip -- a message-passing litmus test of the producer ->
// consumer hand-off the persistent kernels use, run from the test suite
// through mlp_chain_debug_litmus.
//
// The pages give no flag or memory-ordering protocol (the CuSync README
// only says that dependent tiles are synchronized), so this kernel checks
// the one the chain uses, with its own building blocks (chain_device.hpp):
//   publication: plain stores, a workgroup release, a barrier, one agent-
//     scope release store of the flag by thread 0;
//   consumption: one wave polls the flags with relaxed agent-scope loads
//     and back-off (wave_acquire_flags, bounded by a spin limit), takes the
//     hand-off acquire (workgroup scope, or agent scope: `agent`), meets the
//     other waves at an LDS barrier, and every wave then fetches the data
//     with the operand DMA (global_load_lds) into LDS.
// 256 workgroups (one per CU, all resident) run `rounds` rounds in one
// launch.  In round r workgroup b first produces: it writes its share of
// the 8 KB region of pair q = b / 2 (round r, pair q: written exactly once
// per launch, as the intermediate is) and publishes flag (r, b).  Workgroups
// b and b ^ 1 sit on different XCDs (dispatch is round-robin over the 8).
// With `half_lines` each of the two writes one 64-byte half of every
// 128-byte line of the region -- two producers on two XCDs in one line, the
// case of 32-column producer tiles; otherwise each writes 32 whole lines.
// Then b consumes pair (q + 4 k) mod 128 for a k that changes per round:
// one of that pair's producers is on b's own XCD, so b's L2 may hold that
// producer's half of a line when it reads the whole line.  Every 16-byte
// chunk is checked against the value its round, pair and position define;
// mismatches are counted (result[0]) and the first one is recorded
// (result[1..5] = round, consumer, chunk, word read, word expected).  A
// wait that exceeds the spin limit sets result[6] and the kernel carries on,
// so every workgroup exits.
#include <hip/hip_runtime.h>

#include "chain_device.hpp"
#include "chain_launch.h"

namespace mlpc {

constexpr uint32_t LIT_WG = 256;          // workgroups (pairs = 128)
constexpr uint32_t LIT_PAIRS = LIT_WG / 2;
constexpr uint32_t LIT_LINES = 64;        // 128-byte lines per pair region
constexpr uint32_t LIT_REGION = LIT_LINES * 128;

// Value of 32-bit word w of pair q's region in round r (never 0, so memory
// that was never written cannot match).
__device__ __forceinline__ uint32_t lit_value(uint32_t r, uint32_t q, uint32_t w) {
    uint32_t h = (r + 1u) * 0x9E3779B1u ^ (q + 7u) * 0x85EBCA77u ^ (w + 13u) * 0xC2B2AE3Du;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    return h | 1u;
}

__global__ __launch_bounds__(256) void handoff_litmus_kernel(uint8_t* data, uint32_t* flags, uint32_t* res,
                                                              uint32_t rounds, uint32_t half_lines, uint32_t agent,
                                                              uint32_t limit) {
    __shared__ __attribute__((aligned(16))) char buf[LIT_REGION];
    const uint32_t b = blockIdx.x, t = threadIdx.x;
    const uint32_t q = b >> 1, h = b & 1u;
    for (uint32_t r = 0; r < rounds; ++r) {
        // ---- produce: this workgroup's 4 KB of pair q's region
        uint8_t* reg = data + ((size_t)r * LIT_PAIRS + q) * LIT_REGION;
        const uint32_t line = half_lines ? (t >> 2) : h * 32u + (t >> 3);
        const uint32_t off = half_lines ? line * 128u + h * 64u + (t & 3u) * 16u : line * 128u + (t & 7u) * 16u;
        const uint32_t w0 = off / 4u;
        const u32x4 v = u32x4{lit_value(r, q, w0), lit_value(r, q, w0 + 1), lit_value(r, q, w0 + 2),
                              lit_value(r, q, w0 + 3)};
        *reinterpret_cast<u32x4*>(reg + off) = v;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        if (t == 0)
            __hip_atomic_store(flags + r * LIT_WG + b, r + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        // ---- consume pair qc, one of whose producers shares this XCD
        const uint32_t qc = (q + 4u * (1u + r % 31u)) % LIT_PAIRS;
        if ((t >> 6) == 0)
            wave_acquire_flags(flags + r * LIT_WG + 2 * qc, 0, 1, 2, r + 1u, res + 6, limit, agent);
        lds_barrier();
        const uint8_t* src = data + ((size_t)r * LIT_PAIRS + qc) * LIT_REGION;
        const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63u;
#pragma unroll
        for (uint32_t i = 0; i < 2; ++i) {
            const uint32_t c = (wave * 2 + i) * 64 + lane;        // 16-byte chunk of the region
            dma16(src + c * 16, buf + (wave * 2 + i) * 1024);
        }
        ring_barrier<0>();
#pragma unroll
        for (uint32_t i = 0; i < 2; ++i) {
            const uint32_t c = (wave * 2 + i) * 64 + lane;
            const u32x4 got = *reinterpret_cast<const u32x4*>(buf + c * 16);
            for (uint32_t k = 0; k < 4; ++k) {
                const uint32_t want = lit_value(r, qc, c * 4 + k);
                if (got[k] != want) {
                    atomicAdd(res + 0, 1u);
                    if (atomicCAS(res + 1, 0u, r + 1u) == 0u) {
                        res[2] = b;
                        res[3] = c;
                        res[4] = got[k];
                        res[5] = want;
                    }
                    break;
                }
            }
        }
        __syncthreads();     // the LDS buffer is free for the next round
    }
}

}  // namespace mlpc

hipError_t mlpc_litmus(void* data, size_t data_bytes, void* flags, size_t flag_bytes, void* result, int rounds,
                       int half_lines, int agent, uint32_t spin_limit, hipStream_t s) {
    using namespace mlpc;
    if (rounds < 1 || data_bytes < (size_t)rounds * LIT_PAIRS * LIT_REGION ||
        flag_bytes < (size_t)rounds * LIT_WG * 4)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(handoff_litmus_kernel, dim3(LIT_WG), dim3(256), 0, s, static_cast<uint8_t*>(data),
                       static_cast<uint32_t*>(flags), static_cast<uint32_t*>(result), (uint32_t)rounds,
                       (uint32_t)(half_lines != 0), (uint32_t)(agent != 0), spin_limit);
    return hipGetLastError();
}
