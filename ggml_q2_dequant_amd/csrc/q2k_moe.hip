// Expert-routed Q2_K product, matrix-core schedule: routing and row gather.
//
// The operation is the one of the docs.rs source page of mlx-native 0.10.8,
// tests/deepseek_q2_k.rs (fn run_expert, GgmlQuantizedMatmulIdParams, and
// the slotted down-projection test): route r = token * top_k + slot multiplies
// an activation row by expert ids[r]'s weight matrix into output row r.
//
// The matrix-core schedule groups the routes by expert so that each expert's
// weights are decoded once per 128-route tile instead of once per route:
//   1. k_moe_route (one workgroup) counts the routes of every expert, orders
//      them by expert with a stable counting sort (routes of one expert keep
//      increasing r, so the order depends on ids alone) and lists the tiles:
//      runs of at most 128 consecutive rows of one expert, every expert's full
//      128-row tiles first and the partial tiles after them (the GEMM takes
//      them in list order, so the short tiles run last).
//   2. k_moe_gather rounds each route's activation row to bf16 (nearest even)
//      into its row of the expert order, and fills the output rows of routes
//      whose id is out of range (listed after the valid rows of perm) with NaN.
//   3. The GEMM kernel's routed mode (q2k_kernels.hip) multiplies each tile by
//      its expert and writes row p of the order to output row perm[p].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q2k_launch.h"

namespace q2k {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr uint32_t kWave = 64;
constexpr uint32_t kRouteThreads = 1024;
constexpr uint32_t kRouteWaves = kRouteThreads / kWave;

// Exclusive prefix sum of one value per thread over the workgroup, in thread
// order; *total receives the sum of all values.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wsum, uint32_t *total) {
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t incl = v;
#pragma unroll
    for (uint32_t d = 1; d < kWave; d <<= 1) {
        const uint32_t t = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += t;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (uint32_t w = 0; w < kRouteWaves; ++w) {
        const uint32_t s = wsum[w];
        if (w < wave) before += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// One workgroup of 1024 threads. Routes are placed in rounds of 1024 (thread
// t takes route base + t). Within a wavefront, the lanes holding the same
// expert are found by one ballot per bit of the expert id; a lane's row is
// the expert's next free row + the same-expert lanes of lower wavefronts in
// this round + those of lower lanes in its own wavefront. Per round, every
// wavefront records its group sizes tagged with the round number, so stale
// entries of earlier rounds read as zero.
__global__ __launch_bounds__(kRouteThreads) void k_moe_route(const uint32_t *__restrict__ ids, uint32_t routes,
                                                             uint32_t n_experts, uint32_t tiles_max, MoeScratch s,
                                                             int *status) {
    __shared__ uint32_t next[kMoeMaxExperts];             // per expert: count, then next free row
    __shared__ uint32_t first_row[kMoeMaxExperts + 1];
    __shared__ uint32_t first_tile[kMoeMaxExperts + 1];
    __shared__ uint32_t first_part[kMoeMaxExperts + 1];
    __shared__ uint32_t group[kRouteWaves][kMoeMaxExperts];  // (round tag << 16) | lanes of that expert
    __shared__ uint32_t wsum[kRouteWaves];
    __shared__ uint32_t nbad, bad_next;
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

    for (uint32_t i = tid; i < n_experts; i += kRouteThreads) next[i] = 0;
    for (uint32_t i = tid; i < kRouteWaves * kMoeMaxExperts; i += kRouteThreads) (&group[0][0])[i] = 0;
    if (tid == 0) nbad = bad_next = 0;
    __syncthreads();
    uint32_t mybad = 0;
    for (uint32_t r = tid; r < routes; r += kRouteThreads) {
        const uint32_t e = ids[r];
        if (e < n_experts) atomicAdd(&next[e], 1u);
        else ++mybad;
    }
    if (mybad) atomicAdd(&nbad, mybad);
    __syncthreads();

    // Thread e < n_experts holds expert e (n_experts <= kMoeMaxExperts <= 1024).
    const uint32_t c = tid < n_experts ? next[tid] : 0u;
    uint32_t n_valid, n_tiles;
    const uint32_t row = block_exclusive_scan(c, wsum, &n_valid);
    // Tiles: every expert's full tiles first (expert-major), then the partial
    // tiles, so the short ones run last.
    uint32_t n_full, n_part;
    const uint32_t full = c / kMoeTileRows, part = c % kMoeTileRows;
    const uint32_t tile_f = block_exclusive_scan(full, wsum, &n_full);
    const uint32_t tile_p = block_exclusive_scan(part != 0u ? 1u : 0u, wsum, &n_part);
    n_tiles = n_full + n_part;
    if (tid < n_experts) {
        first_row[tid] = row;
        first_tile[tid] = tile_f;
        first_part[tid] = tile_p;
        next[tid] = row;
    }
    if (tid == 0) {
        first_row[n_experts] = n_valid;
        first_tile[n_experts] = n_full;
        first_part[n_experts] = n_part;
    }
    __syncthreads();

    // Tile t < n_full: full tile t - first_tile[e] of the expert e with
    // first_tile[e] <= t < first_tile[e + 1]; tile n_full + u: the partial tile of
    // the expert e with first_part[e] <= u < first_part[e + 1].
    for (uint32_t t = tid; t < tiles_max; t += kRouteThreads) {
        MoeTile mt{0u, 0u, 0u};
        if (t < n_tiles) {
            const bool is_full = t < n_full;
            const uint32_t *first = is_full ? first_tile : first_part;
            const uint32_t key = is_full ? t : t - n_full;
            uint32_t lo = 0, hi = n_experts;  // first[lo] <= key < first[hi]
            while (hi - lo > 1) {
                const uint32_t mid = (lo + hi) / 2;
                if (first[mid] <= key) lo = mid;
                else hi = mid;
            }
            const uint32_t cnt = first_row[lo + 1] - first_row[lo];
            mt.expert = lo;
            if (is_full) {
                mt.p0 = first_row[lo] + (key - first_tile[lo]) * kMoeTileRows;
                mt.count = kMoeTileRows;
            } else {
                mt.p0 = first_row[lo] + cnt / kMoeTileRows * kMoeTileRows;
                mt.count = cnt % kMoeTileRows;
            }
        }
        s.tiles[t] = mt;
    }

    // Stable placement. Key n_experts stands for "no route" (past the end or a bad id).
    const uint32_t nbits = 32u - __builtin_clz(n_experts);
    uint32_t round = 0;
    for (uint32_t base = 0; base < routes; base += kRouteThreads, ++round) {
        const uint32_t r = base + tid;
        uint32_t key = n_experts;
        if (r < routes) {
            const uint32_t e = ids[r];
            if (e < n_experts) key = e;
        }
        uint64_t same = ~0ull;
        for (uint32_t b = 0; b < nbits; ++b) {
            const bool bit = (key >> b) & 1u;
            const uint64_t ones = __ballot(bit);
            same &= bit ? ones : ~ones;
        }
        const uint32_t rank = __popcll(same & ((1ull << lane) - 1ull));
        const uint32_t size = __popcll(same);
        const uint32_t tag = (round + 1u) << 16;
        if (key < n_experts && rank == 0) group[wave][key] = tag | size;
        __syncthreads();
        if (key < n_experts) {
            uint32_t before = 0;
            for (uint32_t w = 0; w < wave; ++w) {
                const uint32_t g = group[w][key];
                if ((g & 0xFFFF0000u) == tag) before += g & 0xFFFFu;
            }
            const uint32_t p = next[key] + before + rank;
            s.perm[p] = r;
        } else if (r < routes) {
            // Routes with a bad id fill the tail of perm (any order).
            s.perm[n_valid + atomicAdd(&bad_next, 1u)] = r;
        }
        __syncthreads();
        if (key < n_experts && rank == 0) atomicAdd(&next[key], size);
        __syncthreads();
    }

    if (tid == 0) {
        s.hdr[0] = n_valid;
        s.hdr[1] = n_tiles;
        s.hdr[2] = nbad;
        s.hdr[3] = 0;
        if (nbad && status) __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

__device__ __forceinline__ bf16x8 to_bf16x8(float4 a, float4 b) {
    bf16x8 v;
    v[0] = static_cast<__bf16>(a.x);
    v[1] = static_cast<__bf16>(a.y);
    v[2] = static_cast<__bf16>(a.z);
    v[3] = static_cast<__bf16>(a.w);
    v[4] = static_cast<__bf16>(b.x);
    v[5] = static_cast<__bf16>(b.y);
    v[6] = static_cast<__bf16>(b.z);
    v[7] = static_cast<__bf16>(b.w);
    return v;
}

// A workgroup per row of the expert order (grid-stride): row p receives
// bf16(x[perm[p] / x_div]); each thread converts chunks of 8 values, loading
// up to kGU chunks before storing any. Then the rows of routes with a bad id
// (perm[n_valid ..]) are filled with NaN in y0 (and y1).
constexpr uint32_t kGU = 4;

__global__ __launch_bounds__(256) void k_moe_gather(const float *__restrict__ x, uint32_t x_div, uint32_t K,
                                                    MoeScratch s, float *y0, float *y1, uint32_t N) {
    const uint32_t n_valid = s.hdr[0], nbad = s.hdr[2], cpr = K / 8, tid = threadIdx.x;
    for (uint32_t p = blockIdx.x; p < n_valid; p += gridDim.x) {
        const uint32_t r = s.perm[p];
        const float4 *src = reinterpret_cast<const float4 *>(x + static_cast<uint64_t>(r / x_div) * K);
        bf16x8 *dst = reinterpret_cast<bf16x8 *>(static_cast<__bf16 *>(s.x_bf16) + static_cast<uint64_t>(p) * K);
        for (uint32_t c0 = 0; c0 < cpr; c0 += kGU * 256u) {
            float4 a[kGU], b[kGU];
#pragma unroll
            for (uint32_t u = 0; u < kGU; ++u) {
                const uint32_t c = c0 + u * 256u + tid;
                if (c < cpr) {
                    a[u] = src[2 * c];
                    b[u] = src[2 * c + 1];
                }
            }
#pragma unroll
            for (uint32_t u = 0; u < kGU; ++u) {
                const uint32_t c = c0 + u * 256u + tid;
                if (c < cpr) dst[c] = to_bf16x8(a[u], b[u]);
            }
        }
    }
    const float nan = __builtin_nanf("");
    for (uint32_t q = blockIdx.x; q < nbad; q += gridDim.x) {
        const uint64_t row = static_cast<uint64_t>(s.perm[n_valid + q]) * N;
        for (uint32_t i = tid; i < N; i += 256u) {
            y0[row + i] = nan;
            if (y1) y1[row + i] = nan;
        }
    }
}

}  // namespace

hipError_t launch_moe_route(const uint32_t *ids, uint32_t routes, uint32_t n_experts, MoeScratch s, int *status,
                            hipStream_t stream) {
    if (n_experts == 0 || n_experts > kMoeMaxExperts || routes == 0 || routes > kMoeMaxRoutes)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(kRouteThreads), 0, stream, ids, routes, n_experts,
                       moe_tiles_max(routes, n_experts), s, status);
    return hipGetLastError();
}

hipError_t launch_moe_gather(const float *x, uint32_t routes, uint32_t x_div, uint32_t K, MoeScratch s, float *y0,
                             float *y1, uint32_t N, hipStream_t stream) {
    const uint32_t grid = routes < 4096u ? routes : 4096u;
    hipLaunchKernelGGL(k_moe_gather, dim3(grid), dim3(256), 0, stream, x, x_div, K, s, y0, y1, N);
    return hipGetLastError();
}

}  // namespace q2k
