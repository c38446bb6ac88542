// GPU first-max argmax and threshold-candidate collect over [n_slots, vocab]
// logits, for gfx950.
//
// What is computed follows the docs.rs source page of mlx-native 0.9.5,
// src/mlx_native/ops/gpu_sample.rs (dispatch_gpu_sample_argmax_candidates and
// its module comment): per slot, the index and value of the first maximum
// (lower index wins ties), every index whose logit is >= top1 - 0.5 (f32), the
// total number of such candidates (which may exceed the capacity `cap`), an
// overflow flag when it does, and up to `cap` candidate ids. The page's own
// kernel collects candidates with an atomic counter, so their order there is
// arbitrary; here they are written in increasing index order, which is one of
// the orders the page allows and makes the output deterministic.
//
// "First maximum" is read as the plain left-to-right scan with a strict
// greater-than: NaN never compares greater, so NaNs are passed over, except
// that a NaN in column 0 is the scan's starting value and stays the answer
// (and then no logit is >= NaN - 0.5, so there are no candidates).
//
// Three launches, each over grid (chunks, slots) with 256 threads:
//   1. per chunk, the first maximum of its non-NaN logits -> partials;
//   2. per chunk, the slot's top1 from all partials (and column 0), then the
//      number of candidates in each quarter of the chunk -> counts; chunk 0
//      writes top1;
//   3. per chunk, each quarter's offset among the slot's candidates (sum of
//      the counts before it), then its candidate ids in index order; chunk 0
//      writes the total and the overflow flag.
// Within a chunk each wavefront walks its quarter 64 columns at a time
// (coalesced); ballots and lane masks rank candidates inside a wavefront.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q2k_launch.h"

namespace q2k {

namespace {

constexpr uint32_t kNone = 0xffffffffu;

struct ArgMax {
    float val;
    uint32_t idx;  // kNone: no non-NaN value seen
};
static_assert(sizeof(ArgMax) == kSampleArgMaxBytes, "workspace sizing assumes 8-byte partials");

// The earlier-index-wins combination of two partial first maxima.
__device__ __forceinline__ ArgMax pick(ArgMax a, ArgMax b) {
    if (a.idx == kNone) return b;
    if (b.idx == kNone) return a;
    if (b.val > a.val) return b;
    if (a.val > b.val) return a;
    return b.idx < a.idx ? b : a;
}

__device__ __forceinline__ ArgMax shfl_xor(ArgMax a, int mask) {
    ArgMax r;
    r.val = __shfl_xor(a.val, mask, 64);
    r.idx = static_cast<uint32_t>(__shfl_xor(static_cast<int>(a.idx), mask, 64));
    return r;
}

__device__ __forceinline__ ArgMax wave_pick(ArgMax a) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) a = pick(a, shfl_xor(a, m));
    return a;
}

// Columns of chunk c of a slot: [c * chunk, min((c + 1) * chunk, vocab)); wave w
// of the workgroup takes the w-th quarter of them.
struct Span {
    uint32_t begin, end;
};

__device__ __forceinline__ Span wave_span(uint32_t c, uint32_t chunk, uint32_t vocab, uint32_t wave) {
    const uint32_t q = chunk / 4;
    const uint32_t b = c * chunk + wave * q;
    Span s;
    s.begin = b < vocab ? b : vocab;
    s.end = b + q < vocab ? b + q : vocab;
    return s;
}

// Walks a wavefront's span 64 columns at a time, 32 steps per round: all 32
// loads of a round are issued before any is used (buffer loads past the row
// return 0 and are flagged out of range), then f(column, value, in_range) runs
// in increasing column order. A quarter of an 8192-column chunk is one round,
// so each pass over the logits waits out one memory latency per wavefront
// (rounds of 8: 18.8 us for 8 x 262144 logits; of 32: 16.2 us).
constexpr uint32_t kRound = 32;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float *row, uint32_t vocab) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), 0, static_cast<int>(vocab * 4u), 0x00020000);
}

template <typename F>
__device__ __forceinline__ void scan_span(__amdgpu_buffer_rsrc_t rs, Span s, uint32_t lane, F f) {
    for (uint32_t i0 = s.begin; i0 < s.end; i0 += 64 * kRound) {
        float v[kRound];
#pragma unroll
        for (uint32_t u = 0; u < kRound; ++u) {
            const uint32_t i = i0 + 64 * u + lane;
            const uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rs, i < s.end ? 4u * i : 0x80000000u, 0, 0);
            v[u] = __builtin_bit_cast(float, e);
        }
#pragma unroll
        for (uint32_t u = 0; u < kRound; ++u) {
            const uint32_t i = i0 + 64 * u + lane;
            f(i, v[u], i < s.end);
        }
    }
}

// Step 1: partial first maximum of each chunk.
__global__ __launch_bounds__(256) void k_argmax_partial(const float *__restrict__ logits, uint32_t vocab,
                                                        uint32_t chunk, ArgMax *__restrict__ part) {
    __shared__ ArgMax red[4];
    const uint32_t slot = blockIdx.y, c = blockIdx.x, lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const float *row = logits + static_cast<uint64_t>(slot) * vocab;
    const Span s = wave_span(c, chunk, vocab, wave);
    ArgMax best{0.0f, kNone};
    scan_span(row_rsrc(row, vocab), s, lane, [&](uint32_t i, float v, bool in) {
        if (in && v == v && (best.idx == kNone || v > best.val)) best = ArgMax{v, i};
    });
    best = wave_pick(best);
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0)
        part[static_cast<uint64_t>(slot) * gridDim.x + c] = pick(pick(red[0], red[1]), pick(red[2], red[3]));
}

// The slot's top1 from its chunk partials (read by the first wavefront).
__device__ __forceinline__ ArgMax slot_top1(const float *row, const ArgMax *part, uint32_t chunks, uint32_t lane) {
    ArgMax b{0.0f, kNone};
    for (uint32_t c = lane; c < chunks; c += 64) b = pick(b, part[c]);
    b = wave_pick(b);
    const float x0 = row[0];
    if (x0 != x0) b = ArgMax{x0, 0};     // the scan starts at column 0 and NaN is never beaten
    if (b.idx == kNone) b = ArgMax{x0, 0};  // unreachable unless column 0 is NaN
    return b;
}

// Step 2: top1 per slot (written by chunk 0) and candidate counts per chunk.
__global__ __launch_bounds__(256) void k_cand_count(const float *__restrict__ logits, uint32_t vocab, uint32_t chunk,
                                                    const ArgMax *__restrict__ part, uint32_t *__restrict__ counts,
                                                    uint32_t *__restrict__ top1_idx, float *__restrict__ top1_val) {
    __shared__ float thr_s;
    const uint32_t slot = blockIdx.y, c = blockIdx.x, chunks = gridDim.x;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const float *row = logits + static_cast<uint64_t>(slot) * vocab;
    if (wave == 0) {
        const ArgMax t = slot_top1(row, part + static_cast<uint64_t>(slot) * chunks, chunks, lane);
        if (lane == 0) {
            thr_s = t.val - 0.5f;
            if (c == 0) {
                top1_idx[slot] = t.idx;
                top1_val[slot] = t.val;
            }
        }
    }
    __syncthreads();
    const float thr = thr_s;
    const Span s = wave_span(c, chunk, vocab, wave);
    uint32_t n = 0;
    scan_span(row_rsrc(row, vocab), s, lane, [&](uint32_t, float v, bool in) { n += __popcll(__ballot(in && v >= thr)); });
    if (lane == 0) counts[(static_cast<uint64_t>(slot) * chunks + c) * 4u + wave] = n;
}

// Step 3: candidate ids in index order, the total and the overflow flag.
__global__ __launch_bounds__(256) void k_cand_collect(const float *__restrict__ logits, uint32_t vocab, uint32_t chunk,
                                                      const ArgMax *__restrict__ part,
                                                      const uint32_t *__restrict__ counts, uint32_t cap,
                                                      uint32_t *__restrict__ cand_count, uint32_t *__restrict__ overflow,
                                                      uint32_t *__restrict__ cand_ids) {
    __shared__ float thr_s;
    __shared__ uint32_t base_s;
    const uint32_t slot = blockIdx.y, c = blockIdx.x, chunks = gridDim.x;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const float *row = logits + static_cast<uint64_t>(slot) * vocab;
    const uint32_t *cnts = counts + static_cast<uint64_t>(slot) * chunks * 4u;
    if (wave == 0) {
        const ArgMax t = slot_top1(row, part + static_cast<uint64_t>(slot) * chunks, chunks, lane);
        uint32_t before = 0, total = 0;
        for (uint32_t k = lane; k < chunks * 4u; k += 64) {
            const uint32_t v = cnts[k];
            total += v;
            if (k < c * 4u) before += v;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            before += static_cast<uint32_t>(__shfl_xor(static_cast<int>(before), m, 64));
            total += static_cast<uint32_t>(__shfl_xor(static_cast<int>(total), m, 64));
        }
        if (lane == 0) {
            thr_s = t.val - 0.5f;
            base_s = before;
            if (c == 0) {
                cand_count[slot] = total;
                overflow[slot] = total > cap ? 1u : 0u;
            }
        }
    }
    const Span s = wave_span(c, chunk, vocab, wave);
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, vocab);
    __syncthreads();
    const float thr = thr_s;
    // The quarters of this chunk before this wavefront's, from the counts of step 2.
    uint32_t pos = base_s;
    for (uint32_t w = 0; w < wave; ++w) pos += cnts[c * 4u + w];
    if (pos >= cap) return;  // this quarter's candidates all fall past the capacity
    uint32_t *out = cand_ids + static_cast<uint64_t>(slot) * cap;
    const uint64_t below = (1ull << lane) - 1ull;
    scan_span(rs, s, lane, [&](uint32_t i, float v, bool in) {
        const bool hit = in && v >= thr;
        const uint64_t m = __ballot(hit);
        const uint32_t r = pos + static_cast<uint32_t>(__popcll(m & below));
        if (hit && r < cap) out[r] = i;
        pos += static_cast<uint32_t>(__popcll(m));
    });
}

}  // namespace

hipError_t launch_argmax_candidates(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                    uint32_t *top1_idx, float *top1_val, uint32_t *cand_count, uint32_t *overflow,
                                    uint32_t *cand_ids, void *workspace, hipStream_t stream) {
    if (n_slots == 0 || n_slots > kMaxGridY) return hipErrorInvalidValue;
    const uint32_t chunk = sample_chunk(vocab);
    const uint32_t chunks = (vocab + chunk - 1) / chunk;
    auto *part = static_cast<ArgMax *>(workspace);
    auto *counts = reinterpret_cast<uint32_t *>(part + static_cast<uint64_t>(n_slots) * chunks);
    const dim3 grid(chunks, n_slots), block(256);
    hipLaunchKernelGGL(k_argmax_partial, grid, block, 0, stream, logits, vocab, chunk, part);
    hipLaunchKernelGGL(k_cand_count, grid, block, 0, stream, logits, vocab, chunk, part, counts, top1_idx, top1_val);
    hipLaunchKernelGGL(k_cand_collect, grid, block, 0, stream, logits, vocab, chunk, part, counts, cap, cand_count,
                       overflow, cand_ids);
    return hipGetLastError();
}

}  // namespace q2k
