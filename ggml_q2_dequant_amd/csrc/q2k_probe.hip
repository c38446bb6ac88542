// Streaming-read ceiling: the cost of only reading a buffer once, with the
// same grid shape as the decode GEMV (a few hundred 256-thread workgroups,
// several 16-byte loads in flight per thread). Benchmarks time it over the
// same cold bytes as a bandwidth-bound kernel, to show how close a transfer
// of that size can get to the HBM peak at all. It computes nothing but an XOR
// of the data per workgroup, stored so that the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q2k_launch.h"

namespace q2k {

namespace {

constexpr uint32_t kReadUnroll = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_read(const u32x4 *__restrict__ data, uint64_t n16, uint32_t *__restrict__ sink) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (uint32_t u = 0; u < kReadUnroll; ++u) v[u] = data[i + u * stride];
#pragma unroll
        for (uint32_t u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= data[i];
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63u) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

uint32_t read_probe_grid(uint64_t bytes) {
    const uint64_t n16 = bytes / 16;
    const uint64_t want = (n16 + 256 * kReadUnroll - 1) / (256 * kReadUnroll);
    return static_cast<uint32_t>(want < kReadProbeMaxGrid ? (want > 0 ? want : 1) : kReadProbeMaxGrid);
}

hipError_t launch_read_probe(const void *data, uint64_t bytes, uint32_t *sink, hipStream_t stream) {
    hipLaunchKernelGGL(k_read, dim3(read_probe_grid(bytes)), dim3(256), 0, stream, static_cast<const u32x4 *>(data),
                       bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace q2k
