// Library-held device scratch for q2k_matmul_noalloc, the matmul entry point
// for callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The matrix-core path (M > 8) stages bf16(x), 2 * M * K bytes, before the
// GEMM reads it. Here that staging lives in `scratch`, a file-scope device
// array of kNoAllocScratchBytes that the code object brings along: every GPU
// the library runs on holds its own copy until the process ends, and no call
// allocates anything. In host code the array's name only stands for it; its
// device address comes from hipGetSymbolAddress, looked up once per device
// (with that device current) on the entry point's first call there and kept.
// Only that address is ever handed to kernels.
//
// Every call on one GPU shares that GPU's array: calls that overlap in time on
// one GPU (two streams, or two host threads) race on it. The kernels overwrite
// all the bytes a call reads, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "q2k_launch.h"

static __device__ __align__(256) uint8_t scratch[q2k::kNoAllocScratchBytes];

namespace q2k {

namespace {

constexpr int kNoAllocMaxDevices = 64;
std::mutex g_noalloc_mu;
void *g_noalloc_ptr[kNoAllocMaxDevices];  // device address of `scratch`, per device ordinal

}  // namespace

hipError_t noalloc_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_noalloc_ptr[dev] = p;
    }
    *out = g_noalloc_ptr[dev];
    return hipSuccess;
}

}  // namespace q2k
