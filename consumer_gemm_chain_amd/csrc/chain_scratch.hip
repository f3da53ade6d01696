// chain_scratch.hip -- the library's static device scratch buffer, for the
// entry point that allocates nothing (mlp_chain_run_noalloc in
// chain_api.cpp), and the kernel that clears its synchronization words.
//
// The buffer is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, from the first use on that device
// until the process ends.  Host code never uses the array's name as a
// device address (in host code it names a host-side stand-in); the address
// of each device's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "chain_launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MLPC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch[MAX_DEVICES];      // each device's address of `scratch` (nullptr: not looked up yet)

// Zero n16 16-byte words at p, and the caller's status word if given.
__global__ void zero_words_kernel(uint4* p, size_t n16, uint32_t* status) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = uint4{0, 0, 0, 0};
    if (status && blockIdx.x == 0 && threadIdx.x == 0) *status = 0u;
}

}  // namespace

hipError_t mlpc_scratch_address(int device, void** ptr) {
    if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // `device` is current
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[device] = p;
    }
    *ptr = g_scratch[device];
    return hipSuccess;
}

hipError_t mlpc_zero_words(void* p, size_t bytes, uint32_t* status, hipStream_t s) {
    if (((uintptr_t)p & 15u) != 0 || (bytes & 15u) != 0) return hipErrorInvalidValue;
    const size_t n16 = bytes / 16;
    const unsigned blocks = (unsigned)(n16 / 256 + 1 < 256 ? n16 / 256 + 1 : 256);
    hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint4*>(p), n16, status);
    return hipGetLastError();
}
