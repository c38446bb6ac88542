// Measurement aid, built as its own library (libq2k_probe.so), not part of
// the Q2_K path or of include/q2k.h: a kernel that only reads a buffer once.
// Benchmarks time it over the same cold bytes as a bandwidth-bound kernel of
// the path, over a range of launch shapes, to show how close a transfer of
// that size can get to the HBM peak at all. It computes nothing but an XOR of
// the data per workgroup, stored so that the loads cannot be dropped.
//
// C entry point (plain device pointers, no torch types):
//   int q2k_probe_read(const void *data, size_t bytes, uint32_t *sink, size_t sink_elems,
//                      uint32_t grid, uint32_t unroll, void *stream);
//     data   device memory, 16-byte aligned; bytes a positive multiple of 16.
//     grid   workgroups of 256 threads, 1 .. 16384; 0 picks the default shape
//            (enough workgroups that each thread issues `unroll` 16-byte loads
//            per round, at most 2048).
//     unroll 16-byte loads a thread keeps in flight per round: 1, 2, 4, 8 or 16.
//     sink   device u32 [sink_elems], one word per workgroup (sink_elems >= grid);
//            must not overlap data.
//   Returns 0 once enqueued on `stream`, 1 for a bad argument, 3 if the launch
//   failed. Allocates nothing.
//   uint32_t q2k_probe_default_grid(size_t bytes, uint32_t unroll);
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr uint32_t kProbeMaxGrid = 16384;
constexpr uint32_t kProbeDefaultMaxGrid = 2048;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <uint32_t U>
__global__ __launch_bounds__(256) void k_read(const u32x4 *__restrict__ data, uint64_t n16, uint32_t *__restrict__ sink) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) v[u] = data[i + u * stride];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) acc ^= v[u];
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

bool overlap(const void *p, uint64_t n, const void *q, uint64_t m) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return n != 0 && m != 0 && a < b + m && b < a + n;
}

}  // namespace

extern "C" {

uint32_t q2k_probe_default_grid(size_t bytes, uint32_t unroll) {
    const uint64_t n16 = bytes / 16, per = 256ull * (unroll ? unroll : 1);
    const uint64_t want = (n16 + per - 1) / per;
    return static_cast<uint32_t>(want < kProbeDefaultMaxGrid ? (want > 0 ? want : 1) : kProbeDefaultMaxGrid);
}

int q2k_probe_read(const void *data, size_t bytes, uint32_t *sink, size_t sink_elems, uint32_t grid, uint32_t unroll,
                   void *stream) {
    if (!data || !sink || bytes == 0 || bytes % 16 != 0) return 1;
    if ((reinterpret_cast<uintptr_t>(data) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return 1;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16) return 1;
    if (grid == 0) grid = q2k_probe_default_grid(bytes, unroll);
    if (grid > kProbeMaxGrid || sink_elems < grid) return 1;
    if (overlap(sink, 4ull * grid, data, bytes)) return 1;
    const auto *d = static_cast<const u32x4 *>(data);
    const auto st = static_cast<hipStream_t>(stream);
    const uint64_t n16 = bytes / 16;
    switch (unroll) {
        case 1: hipLaunchKernelGGL(k_read<1>, dim3(grid), dim3(256), 0, st, d, n16, sink); break;
        case 2: hipLaunchKernelGGL(k_read<2>, dim3(grid), dim3(256), 0, st, d, n16, sink); break;
        case 4: hipLaunchKernelGGL(k_read<4>, dim3(grid), dim3(256), 0, st, d, n16, sink); break;
        case 8: hipLaunchKernelGGL(k_read<8>, dim3(grid), dim3(256), 0, st, d, n16, sink); break;
        default: hipLaunchKernelGGL(k_read<16>, dim3(grid), dim3(256), 0, st, d, n16, sink); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
