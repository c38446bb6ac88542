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
// Two launches. The first reads the logits once, grid (chunks, slots) with
// 256 threads: per chunk, the first maximum of its non-NaN logits (a partial),
// and its local candidates, the logits >= (chunk maximum) - 0.5, counted and
// the first kSampleLocalCap of them kept (index and value, in index order).
// The slot's maximum is at least the chunk's, and f32 rounding of x - 0.5 is
// monotonic, so every candidate of the slot is a local candidate of its chunk.
// The second, one workgroup per slot, takes top1 from the partials (and
// column 0), counts each chunk's candidates among its kept ones (rescanning
// the chunk's logits only when it had more local candidates than it kept),
// and writes the first cap candidate ids in index order, the total and the
// overflow flag. Within a chunk each wavefront walks its quarter 64 columns
// at a time (coalesced); ballots and lane masks rank candidates inside a
// wavefront. For 8 x 262144 Gaussian logits the two take 10.9 us per call,
// against 14.7 us for three passes (maximum, count, collect) that each read
// the logits.
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

// Walks a wavefront's span 64 columns at a time, R steps per round: all R
// loads of a round are issued before any is used (buffer loads past the row
// return 0 and are flagged out of range), then f(column, value, in_range) runs
// in increasing column order, so each pass over the logits waits out one
// memory latency per round (in an earlier three-pass form of this call,
// rounds of 8 took 18.8 us for 8 x 262144 logits and rounds of 32 16.2 us).
// The scan walks chunks longer than 4096 logits (vocabularies above 2^18) in
// rounds of 32.
constexpr uint32_t kRound = 32;

// Chunks of 4096 logits (the minimum) take the one-round form instead: a
// wavefront's quarter is 16 steps, all loaded up front and held in registers
// for every walk (round_first_max and below). 4096-logit chunks give 512
// workgroups for 8 x 262144 logits: 10.9 us per call, against 12.2 us with
// 8192-logit chunks (256 workgroups, 32 steps) and 13.8 us with 2048 (the
// finish pass then holds twice the chunks). The finish pass's rare rescans
// of whole chunks also go in rounds of 16: rounds of 32 there cost its
// common path registers and 0.6 us per call.
constexpr uint32_t kOneRoundSteps = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float *row, uint32_t vocab) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), 0, static_cast<int>(vocab * 4u), 0x00020000);
}

template <uint32_t R, typename F>
__device__ __forceinline__ void scan_span(__amdgpu_buffer_rsrc_t rs, Span s, uint32_t lane, F f) {
    for (uint32_t i0 = s.begin; i0 < s.end; i0 += 64 * R) {
        float v[R];
#pragma unroll
        for (uint32_t u = 0; u < R; ++u) {
            const uint32_t i = i0 + 64 * u + lane;
            const uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rs, i < s.end ? 4u * i : 0x80000000u, 0, 0);
            v[u] = __builtin_bit_cast(float, e);
        }
#pragma unroll
        for (uint32_t u = 0; u < R; ++u) {
            const uint32_t i = i0 + 64 * u + lane;
            f(i, v[u], i < s.end);
        }
    }
}

// Local candidates of one chunk, kept by the scan: index and value.
struct Cand {
    uint32_t idx;
    float val;
};
static_assert(sizeof(Cand) == kSampleCandBytes, "workspace sizing assumes 8-byte candidates");

// Where the scan leaves a slot's chunks in the workspace: partials, local
// candidate counts, kept candidates.
struct SampleWs {
    ArgMax *part;    // [slots * chunks]
    uint32_t *nloc;  // [slots * chunks]
    Cand *cand;      // [slots * chunks * kSampleLocalCap]
};

inline SampleWs sample_ws(void *ws, uint32_t n_slots, uint32_t chunks) {
    const uint64_t pc = static_cast<uint64_t>(n_slots) * chunks;
    SampleWs w;
    w.part = static_cast<ArgMax *>(ws);
    w.cand = reinterpret_cast<Cand *>(w.part + pc);
    w.nloc = reinterpret_cast<uint32_t *>(w.cand + pc * kSampleLocalCap);
    return w;
}

// Wavefront reductions without a trip through LDS: within each row of 16
// lanes by DPP moves (quad xor 1, quad xor 2, row rotations by 4 and 8), then
// across rows by the gfx950 lane swaps (rows 0/1 and 2/3, then the halves),
// which hand every lane of a pair both partners' values.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ ArgMax dpp_move(ArgMax a) {
    return ArgMax{dpp_move<CTRL>(a.val),
                  static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(a.idx), CTRL, 0xF, 0xF, false))};
}

// The values of the two rows (16 lanes) or halves (32 lanes) that a lane swap
// pairs, at the lane's position, in every lane of either.
__device__ __forceinline__ void swap16(uint32_t v, uint32_t *even, uint32_t *odd) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    *even = r[0];
    *odd = r[1];
}

__device__ __forceinline__ void swap32(uint32_t v, uint32_t *lo, uint32_t *hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    *lo = r[0];
    *hi = r[1];
}

// The wavefront's first maximum (pick over all 64 lanes) in every lane, by the
// same moves as wave_fmax; pick is a maximum under a total order, so the
// order of combination does not matter.
__device__ __forceinline__ ArgMax wave_pick(ArgMax a) {
    a = pick(a, dpp_move<0xB1>(a));
    a = pick(a, dpp_move<0x4E>(a));
    a = pick(a, dpp_move<0x124>(a));
    a = pick(a, dpp_move<0x128>(a));
    uint32_t v0, v1, i0, i1;
    swap16(__builtin_bit_cast(uint32_t, a.val), &v0, &v1);
    swap16(a.idx, &i0, &i1);
    a = pick(ArgMax{__builtin_bit_cast(float, v0), i0}, ArgMax{__builtin_bit_cast(float, v1), i1});
    swap32(__builtin_bit_cast(uint32_t, a.val), &v0, &v1);
    swap32(a.idx, &i0, &i1);
    return pick(ArgMax{__builtin_bit_cast(float, v0), i0}, ArgMax{__builtin_bit_cast(float, v1), i1});
}

// The largest non-NaN value over the wavefront in every lane (NaN if all are
// NaN; max ignores NaN).
__device__ __forceinline__ float wave_fmax(float m) {
    m = __builtin_fmaxf(m, dpp_move<0xB1>(m));   // quad_perm [1,0,3,2]
    m = __builtin_fmaxf(m, dpp_move<0x4E>(m));   // quad_perm [2,3,0,1]
    m = __builtin_fmaxf(m, dpp_move<0x124>(m));  // row_ror 4
    m = __builtin_fmaxf(m, dpp_move<0x128>(m));  // row_ror 8
    uint32_t e, o;
    swap16(__builtin_bit_cast(uint32_t, m), &e, &o);
    m = __builtin_fmaxf(__builtin_bit_cast(float, e), __builtin_bit_cast(float, o));
    swap32(__builtin_bit_cast(uint32_t, m), &e, &o);
    return __builtin_fmaxf(__builtin_bit_cast(float, e), __builtin_bit_cast(float, o));
}

// The wavefront's first maximum over its quarter when the quarter is one
// round held in registers (v[u] is column begin + 64 u + lane, NaN past the
// row): the largest non-NaN value M (max ignores NaN), then the lowest
// column holding a value equal to M, and that column's own value (so +0 and
// -0 keep their bits).
__device__ __forceinline__ ArgMax round_first_max(const float (&v)[kOneRoundSteps], uint32_t begin, uint32_t lane) {
    float m = v[0];
#pragma unroll
    for (uint32_t u = 1; u < kOneRoundSteps; ++u) m = __builtin_fmaxf(m, v[u]);
    m = wave_fmax(m);
    if (m != m) return ArgMax{0.0f, kNone};  // no non-NaN value in the quarter
    // Steps in column order; the first whose ballot finds M holds the answer in its lowest such lane.
#pragma unroll
    for (uint32_t u = 0; u < kOneRoundSteps; ++u) {
        const uint64_t b = __ballot(v[u] == m);
        if (b != 0) {
            const uint32_t l = static_cast<uint32_t>(__builtin_ctzll(b));
            const float val = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[u]), l));
            return ArgMax{val, begin + 64u * u + l};
        }
    }
    return ArgMax{0.0f, kNone};  // unreachable: M is one of the values
}

// Pass 1: per chunk, the partial first maximum and the local candidates. The
// wavefront's quarter is walked up to three times (maximum, count, collect);
// kOneRound: the quarter is a single round, whose values stay in registers.
template <bool kOneRound>
__global__ __launch_bounds__(256) void k_sample_scan(const float *__restrict__ logits, uint32_t vocab, uint32_t chunk,
                                                     SampleWs ws) {
    __shared__ ArgMax red[4];
    __shared__ uint32_t cnt[4];
    const uint32_t slot = blockIdx.y, c = blockIdx.x, chunks = gridDim.x;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const float *row = logits + static_cast<uint64_t>(slot) * vocab;
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, vocab);
    const Span s = wave_span(c, chunk, vocab, wave);
    const uint64_t below = (1ull << lane) - 1ull;
    const uint64_t pc = static_cast<uint64_t>(slot) * chunks + c;
    Cand *out = ws.cand + pc * kSampleLocalCap;
    float v1[kOneRoundSteps];  // kOneRound: the wavefront's whole quarter, NaN past the row
    ArgMax best{0.0f, kNone};
    if constexpr (kOneRound) {
        // Column begin + 64 u + lane at byte offset 4 (begin + lane) + 256 u (the step in the scalar offset);
        // past the quarter it is another wavefront's logit or, past the row, zero: NaN either way here.
        // All loads are issued before the first is used (left free, the scheduler may start the maximum
        // after some of them and issue the rest a memory latency later).
        const uint32_t len = s.end - s.begin;
        uint32_t e[kOneRoundSteps];
#pragma unroll
        for (uint32_t u = 0; u < kOneRoundSteps; ++u)
            e[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * (s.begin + lane), 256u * u, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t u = 0; u < kOneRoundSteps; ++u) v1[u] = 64u * u + lane < len ? __builtin_bit_cast(float, e[u]) : __builtin_nanf("");
        best = round_first_max(v1, s.begin, lane);
    } else {
        scan_span<kRound>(rs, s, lane, [&](uint32_t i, float v, bool in) {
            if (in && v == v && (best.idx == kNone || v > best.val)) best = ArgMax{v, i};
        });
        best = wave_pick(best);
    }
    if (lane == 0) red[wave] = best;
    __syncthreads();
    const ArgMax cm = pick(pick(red[0], red[1]), pick(red[2], red[3]));
    if (threadIdx.x == 0) ws.part[pc] = cm;
    if (cm.idx == kNone) {  // no non-NaN logit in the chunk: no candidates
        if (threadIdx.x == 0) ws.nloc[pc] = 0;
        return;
    }
    const float thr = cm.val - 0.5f;
    uint32_t n = 0;
    if constexpr (kOneRound) {
#pragma unroll
        for (uint32_t u = 0; u < kOneRoundSteps; ++u) n += static_cast<uint32_t>(__popcll(__ballot(v1[u] >= thr)));
    } else {
        scan_span<kRound>(rs, s, lane, [&](uint32_t, float v, bool in) { n += static_cast<uint32_t>(__popcll(__ballot(in && v >= thr))); });
    }
    if (lane == 0) cnt[wave] = n;
    __syncthreads();
    uint32_t pos = 0;
    for (uint32_t w = 0; w < wave; ++w) pos += cnt[w];
    if (threadIdx.x == 0) ws.nloc[pc] = (cnt[0] + cnt[1]) + (cnt[2] + cnt[3]);
    if (pos >= kSampleLocalCap || n == 0) return;
    if constexpr (kOneRound) {
#pragma unroll
        for (uint32_t u = 0; u < kOneRoundSteps; ++u) {
            const uint64_t mk = __ballot(v1[u] >= thr);
            if (mk != 0) {  // uniform: most steps of a quarter hold no candidate
                const bool hit = (mk >> lane) & 1ull;
                const uint32_t r = pos + static_cast<uint32_t>(__popcll(mk & below));
                if (hit && r < kSampleLocalCap) out[r] = Cand{s.begin + 64 * u + lane, v1[u]};
                pos += static_cast<uint32_t>(__popcll(mk));
            }
        }
    } else {
        scan_span<kRound>(rs, s, lane, [&](uint32_t i, float v, bool in) {
            const bool hit = in && v >= thr;
            const uint64_t m = __ballot(hit);
            const uint32_t r = pos + static_cast<uint32_t>(__popcll(m & below));
            if (hit && r < kSampleLocalCap) out[r] = Cand{i, v};
            pos += static_cast<uint32_t>(__popcll(m));
        });
    }
}

// The slot's top1 from its chunk partials, lane c holding chunk c's (c < chunks <= 64), and column 0.
__device__ __forceinline__ ArgMax slot_top1(ArgMax own, float x0, uint32_t chunks, uint32_t lane) {
    ArgMax b = lane < chunks ? own : ArgMax{0.0f, kNone};
    b = wave_pick(b);
    if (x0 != x0) b = ArgMax{x0, 0};     // the scan starts at column 0 and NaN is never beaten
    if (b.idx == kNone) b = ArgMax{x0, 0};  // unreachable unless column 0 is NaN
    return b;
}

// Pass 2: one workgroup per slot. Wavefront w takes chunks w, w + 4, ... (at
// most kSampleMaxChunks / 4 of them): it loads their local counts and kept
// candidates (lane j: the j-th kept one) unconditionally, from clamped
// addresses, so they are all in flight together and the pass waits out one
// memory latency rather than one per chunk. A chunk with more local candidates
// than were kept is rescanned from the logits, in loops of their own (rare:
// many logits within 0.5 of a chunk's maximum).
constexpr uint32_t kFinishPer = kSampleMaxChunks / 4;
static_assert(kSampleLocalCap == 64, "one kept candidate per lane");

__global__ __launch_bounds__(256) void k_sample_finish(const float *__restrict__ logits, uint32_t vocab, uint32_t chunk,
                                                       uint32_t chunks, SampleWs ws, uint32_t cap,
                                                       uint32_t *__restrict__ top1_idx, float *__restrict__ top1_val,
                                                       uint32_t *__restrict__ cand_count,
                                                       uint32_t *__restrict__ overflow, uint32_t *__restrict__ cand_ids) {
    __shared__ float thr_s;
    __shared__ uint32_t sc[kSampleMaxChunks];  // candidates of the slot per chunk, then their exclusive prefix
    const uint32_t slot = blockIdx.x;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const float *row = logits + static_cast<uint64_t>(slot) * vocab;
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, vocab);
    const uint64_t p0 = static_cast<uint64_t>(slot) * chunks;
    uint32_t nl[kFinishPer];
    Cand kc[kFinishPer];
    // Every load of the pass up front (clamped addresses, nothing conditional), so it waits out one memory
    // latency: the partials (one chunk per lane), column 0, the counts and kept candidates.
    static_assert(kSampleMaxChunks <= 64, "one chunk partial per lane");
    const ArgMax own = ws.part[p0 + min(lane, chunks - 1u)];
    const float x0 = row[0];
#pragma unroll
    for (uint32_t q = 0; q < kFinishPer; ++q) {
        const uint32_t c = min(wave + 4u * q, chunks - 1u);
        nl[q] = ws.nloc[p0 + c];
        kc[q] = ws.cand[(p0 + c) * kSampleLocalCap + lane];
    }
    if (wave == 0) {
        const ArgMax t = slot_top1(own, x0, chunks, lane);
        if (lane == 0) {
            thr_s = t.val - 0.5f;
            top1_idx[slot] = t.idx;
            top1_val[slot] = t.val;
        }
    }
    __syncthreads();
    const float thr = thr_s;
    const uint64_t below = (1ull << lane) - 1ull;
    // The whole chunk c, walked by one wavefront in order.
    auto chunk_span = [&](uint32_t c) __attribute__((always_inline)) {
        const uint32_t b = c * chunk;
        return Span{b, b + chunk < vocab ? b + chunk : vocab};
    };
    uint64_t hits[kFinishPer];
    uint32_t rescan = 0;  // bit q: chunk wave + 4 q had more local candidates than were kept
#pragma unroll
    for (uint32_t q = 0; q < kFinishPer; ++q) {
        const uint32_t c = wave + 4u * q;
        const bool kept = c < chunks && nl[q] <= kSampleLocalCap;
        if (c < chunks && !kept) rescan |= 1u << q;
        hits[q] = __ballot(kept && lane < nl[q] && kc[q].val >= thr);
        if (lane == 0 && kept) sc[c] = static_cast<uint32_t>(__popcll(hits[q]));
    }
    rescan = __builtin_amdgcn_readfirstlane(rescan);
#pragma nounroll
    for (uint32_t todo = rescan; todo != 0; todo &= todo - 1u) {
        const uint32_t c = wave + 4u * static_cast<uint32_t>(__builtin_ctz(todo));
        uint32_t n = 0;
        scan_span<kOneRoundSteps>(rs, chunk_span(c), lane, [&](uint32_t, float v, bool in) {
            n += static_cast<uint32_t>(__popcll(__ballot(in && v >= thr)));
        });
        if (lane == 0) sc[c] = n;
    }
    __syncthreads();
    // Exclusive prefix of the chunk counts (one per lane of wavefront 0) and the total.
    if (wave == 0) {
        const uint32_t own = lane < chunks ? sc[lane] : 0u;
        uint32_t v = own;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t u = static_cast<uint32_t>(__shfl_up(static_cast<int>(v), d, 64));
            if (lane >= static_cast<uint32_t>(d)) v += u;
        }
        if (lane < chunks) sc[lane] = v - own;
        if (lane == 63) {
            cand_count[slot] = v;
            overflow[slot] = v > cap ? 1u : 0u;
        }
    }
    __syncthreads();
    uint32_t *out = cand_ids + static_cast<uint64_t>(slot) * cap;
#pragma unroll
    for (uint32_t q = 0; q < kFinishPer; ++q) {
        const uint32_t c = wave + 4u * q;
        if (c < chunks && nl[q] <= kSampleLocalCap && hits[q] != 0) {
            const uint32_t pos = sc[c];
            const bool hit = (hits[q] >> lane) & 1ull;
            const uint32_t r = pos + static_cast<uint32_t>(__popcll(hits[q] & below));
            if (hit && r < cap) out[r] = kc[q].idx;
        }
    }
#pragma nounroll
    for (uint32_t todo = rescan; todo != 0; todo &= todo - 1u) {
        const uint32_t c = wave + 4u * static_cast<uint32_t>(__builtin_ctz(todo));
        uint32_t pos = sc[c];
        if (pos >= cap) continue;
        scan_span<kOneRoundSteps>(rs, chunk_span(c), lane, [&](uint32_t i, float v, bool in) {
            const bool hit = in && v >= thr;
            const uint64_t m = __ballot(hit);
            const uint32_t r = pos + static_cast<uint32_t>(__popcll(m & below));
            if (hit && r < cap) out[r] = i;
            pos += static_cast<uint32_t>(__popcll(m));
        });
    }
}

}  // namespace

hipError_t launch_argmax_candidates(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                    uint32_t *top1_idx, float *top1_val, uint32_t *cand_count, uint32_t *overflow,
                                    uint32_t *cand_ids, void *workspace, hipStream_t stream) {
    if (n_slots == 0 || n_slots > kMaxGridY) return hipErrorInvalidValue;
    const uint32_t chunk = sample_chunk(vocab);
    const uint32_t chunks = (vocab + chunk - 1) / chunk;
    const SampleWs ws = sample_ws(workspace, n_slots, chunks);
    const dim3 grid(chunks, n_slots), block(256);
    if (chunk / 4 <= 64 * kOneRoundSteps)
        hipLaunchKernelGGL(k_sample_scan<true>, grid, block, 0, stream, logits, vocab, chunk, ws);
    else
        hipLaunchKernelGGL(k_sample_scan<false>, grid, block, 0, stream, logits, vocab, chunk, ws);
    hipLaunchKernelGGL(k_sample_finish, dim3(n_slots), block, 0, stream, logits, vocab, chunk, chunks, ws, cap,
                       top1_idx, top1_val, cand_count, overflow, cand_ids);
    return hipGetLastError();
}

}  // namespace q2k
