// Host-memory stand-ins for the HIP runtime calls and kernel launches that the
// C ABI layer (q2k_api.cpp) makes, so that layer can be built with g++ and
// AddressSanitizer/UBSan and driven without a GPU.
//
// "Device" memory here is host heap memory: hipMalloc returns a 256-byte
// aligned block of exactly the requested size, so a stray byte past a
// workspace is a heap-buffer-overflow that ASan reports. Each launch stub
// touches every byte its kernel reads (one load each) and writes every byte
// it writes, using the kernel's documented layout (q2k_launch.h and the
// kernels' own comments), not the sizing functions of the ABI layer. Given
// host buffers of exactly the sizes the header states, any call that hands a
// kernel a pointer, size or scratch layout beyond its buffer faults under
// ASan. Nothing is computed: outputs are filled with a marker value.
//
// Also exported for drivers (extern "C"):
//   stub_set_capturing(int)   makes hipStreamIsCapturing report an active capture
//   stub_fail_gather_done(int) makes the gather's completion launch fail
//   stub_launches()           number of launch stubs run so far
//   stub_mallocs()            number of hipMalloc calls so far
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "q2k_launch.h"

namespace {

std::atomic<int> g_capturing{0};
std::atomic<int> g_fail_done{0};
std::atomic<unsigned long long> g_launches{0};
std::atomic<unsigned long long> g_mallocs{0};

thread_local volatile uint8_t g_sink;

void read_bytes(const void *p, uint64_t n) {
    const auto *b = static_cast<const volatile uint8_t *>(p);
    uint8_t acc = 0;
    for (uint64_t i = 0; i < n; ++i) acc ^= b[i];
    g_sink = acc;
}

void write_bytes(void *p, uint64_t n) {
    auto *b = static_cast<volatile uint8_t *>(p);
    for (uint64_t i = 0; i < n; ++i) b[i] = 0xA5;
}

uint64_t row_bytes(uint32_t K) { return static_cast<uint64_t>(K / q2k::kQK) * q2k::kBlockBytes; }

hipError_t launched() {
    ++g_launches;
    return hipSuccess;
}

}  // namespace

extern "C" {

void stub_set_capturing(int on) { g_capturing = on; }
void stub_fail_gather_done(int on) { g_fail_done = on; }
unsigned long long stub_launches(void) { return g_launches; }
unsigned long long stub_mallocs(void) { return g_mallocs; }

hipError_t hipGetDevice(int *deviceId) {
    *deviceId = 0;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t) { return "stub runtime error"; }

hipError_t hipMalloc(void **ptr, size_t size) {
    ++g_mallocs;
    *ptr = nullptr;
    return posix_memalign(ptr, 256, size ? size : 1) == 0 ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipHostMalloc(void **ptr, size_t size, unsigned int) {
    *ptr = std::calloc(1, size ? size : 1);
    return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipHostGetDevicePointer(void **devPtr, void *hstPtr, unsigned int) {
    *devPtr = hstPtr;
    return hipSuccess;
}

hipError_t hipFree(void *ptr) {
    std::free(ptr);
    return hipSuccess;
}

hipError_t hipMemset(void *dst, int value, size_t sizeBytes) {
    std::memset(dst, value, sizeBytes);
    return hipSuccess;
}

hipError_t hipDeviceSynchronize(void) { return hipSuccess; }

hipError_t hipHostFree(void *ptr) {
    std::free(ptr);
    return hipSuccess;
}

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *status) {
    *status = g_capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

}  // extern "C"

namespace q2k {

hipError_t launch_dequantize(const uint8_t *blocks, uint64_t nblocks, float *out, hipStream_t) {
    read_bytes(blocks, nblocks * kBlockBytes);
    write_bytes(out, nblocks * kQK * 4);
    return launched();
}

hipError_t launch_gather(const uint8_t *table, const uint32_t *ids, float *out, uint32_t vocab,
                         uint32_t blocks_per_row, uint32_t n_tokens, int *status, int bad_value, hipStream_t) {
    // Each token's row of blocks_per_row blocks, or a NaN row and the status
    // word for an id >= vocab.
    const uint64_t rb = static_cast<uint64_t>(blocks_per_row) * kBlockBytes;
    for (uint32_t t = 0; t < n_tokens; ++t) {
        const uint32_t id = ids[t];
        if (id < vocab)
            read_bytes(table + id * rb, rb);
        else
            *status = bad_value;
        write_bytes(out + static_cast<uint64_t>(t) * blocks_per_row * kQK, 4ull * blocks_per_row * kQK);
    }
    return launched();
}

hipError_t launch_gather_done(int *status, int seq, int *host_word, hipStream_t) {
    if (g_fail_done) return hipErrorLaunchFailure;
    // Stands in for the one-thread kernel: clears the marker and publishes the outcome at once.
    const int v = __atomic_load_n(status, __ATOMIC_RELAXED);
    __atomic_store_n(status, 0, __ATOMIC_RELAXED);
    __atomic_store_n(host_word, (seq << 2) | 2 | (v == seq ? 1 : 0), __ATOMIC_RELEASE);
    return launched();
}

hipError_t launch_gemv(const float *x, const uint8_t *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                       uint32_t batches, hipStream_t) {
    if (M == 0 || M > kGemvMaxM || batches == 0 || batches > kMaxGridY) return hipErrorInvalidValue;
    read_bytes(x, 4ull * batches * M * K);
    read_bytes(w, static_cast<uint64_t>(batches) * N * row_bytes(K));
    write_bytes(y, 4ull * batches * M * N);
    return launched();
}

hipError_t launch_gemm_mfma(const float *x, const uint8_t *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                            void *x_bf16, hipStream_t) {
    if (reinterpret_cast<uintptr_t>(x_bf16) & 15u) return hipErrorInvalidValue;
    read_bytes(x, 4ull * M * K);
    write_bytes(x_bf16, 2ull * M * K);   // the pre-pass: bf16(x)
    read_bytes(x_bf16, 2ull * M * K);    // the GEMM reads it back
    read_bytes(w, static_cast<uint64_t>(N) * row_bytes(K));
    write_bytes(y, 4ull * M * N);
    return launched();
}

hipError_t noalloc_scratch(void **out) {
    // The library's file-scope device array, as one host block of its size.
    static void *block = [] {
        void *p = nullptr;
        return posix_memalign(&p, 256, kNoAllocScratchBytes) == 0 ? p : nullptr;
    }();
    *out = block;
    return block ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t launch_argmax_candidates(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                    uint32_t *top1_idx, float *top1_val, uint32_t *cand_count, uint32_t *overflow,
                                    uint32_t *cand_ids, void *workspace, hipStream_t) {
    if (n_slots == 0 || n_slots > kMaxGridY) return hipErrorInvalidValue;
    if (reinterpret_cast<uintptr_t>(workspace) & 7u) return hipErrorInvalidValue;
    // Workspace layout of the two launches, per (slot, chunk): an 8-byte
    // partial (value, index) each, then kSampleLocalCap 8-byte kept candidates
    // each, then a u32 local candidate count each. The scan writes them all;
    // the finish pass reads them all back.
    const uint32_t chunk = sample_chunk(vocab);
    const uint64_t chunks = (vocab + chunk - 1) / chunk;
    const uint64_t parts = static_cast<uint64_t>(n_slots) * chunks;
    const uint64_t bytes = parts * (8 + 8ull * kSampleLocalCap + 4);
    read_bytes(logits, 4ull * n_slots * vocab);
    write_bytes(workspace, bytes);
    read_bytes(workspace, bytes);
    write_bytes(top1_idx, 4ull * n_slots);
    write_bytes(top1_val, 4ull * n_slots);
    write_bytes(cand_count, 4ull * n_slots);
    write_bytes(overflow, 4ull * n_slots);
    write_bytes(cand_ids, 4ull * n_slots * cap);
    return launched();
}

hipError_t launch_moe_gemv(const float *x, const uint8_t *w, const uint32_t *ids, float *y, uint32_t routes,
                           uint32_t x_div, uint32_t N, uint32_t K, uint32_t n_experts, uint64_t expert_stride,
                           int *status, hipStream_t) {
    // Route r: activation row r / x_div times expert ids[r]'s N rows into
    // output row r; a bad id gives a NaN row and sets *status when given.
    for (uint32_t r = 0; r < routes; ++r) {
        const uint32_t e = ids[r];
        if (e < n_experts) {
            read_bytes(x + static_cast<uint64_t>(r / x_div) * K, 4ull * K);
            read_bytes(w + e * expert_stride, static_cast<uint64_t>(N) * row_bytes(K));
        } else if (status) {
            *status = 1;
        }
        write_bytes(y + static_cast<uint64_t>(r) * N, 4ull * N);
    }
    return launched();
}

hipError_t launch_moe_route(const uint32_t *ids, uint32_t routes, uint32_t n_experts, MoeScratch s, int *status,
                            hipStream_t) {
    if (n_experts == 0 || n_experts > kMoeMaxExperts || routes == 0 || routes > kMoeMaxRoutes)
        return hipErrorInvalidValue;
    read_bytes(ids, 4ull * routes);
    // Header (valid routes, tiles used, bad routes), the expert order of all
    // routes, and one tile record per 128-row run of one expert.
    uint32_t valid = 0, bad = 0, tiles = 0;
    uint32_t count[kMoeMaxExperts] = {};
    for (uint32_t r = 0; r < routes; ++r) {
        if (ids[r] < n_experts)
            ++count[ids[r]], ++valid;
        else
            ++bad;
    }
    for (uint32_t e = 0; e < n_experts; ++e) tiles += (count[e] + kMoeTileRows - 1) / kMoeTileRows;
    write_bytes(s.hdr, 16);
    s.hdr[0] = valid;
    s.hdr[1] = tiles;
    s.hdr[2] = bad;
    s.hdr[3] = 0;
    uint32_t p = 0;
    for (uint32_t e = 0; e < n_experts; ++e)
        for (uint32_t r = 0; r < routes; ++r)
            if (ids[r] == e) s.perm[p++] = r;
    for (uint32_t r = 0; r < routes; ++r)
        if (ids[r] >= n_experts) s.perm[p++] = r;
    uint32_t t = 0, p0 = 0;
    for (uint32_t e = 0; e < n_experts; ++e) {
        for (uint32_t done = 0; done < count[e]; done += kMoeTileRows) {
            const uint32_t c = count[e] - done < kMoeTileRows ? count[e] - done : kMoeTileRows;
            s.tiles[t++] = MoeTile{e, p0 + done, c};
        }
        p0 += count[e];
    }
    if (bad && status) *status = 1;
    return launched();
}

hipError_t launch_moe_gather(const float *x, uint32_t routes, uint32_t x_div, uint32_t K, MoeScratch s, float *y0,
                             float *y1, uint32_t N, hipStream_t) {
    const uint32_t valid = s.hdr[0];
    auto *xb = static_cast<uint8_t *>(s.x_bf16);
    for (uint32_t p = 0; p < routes; ++p) {
        const uint32_t r = s.perm[p];
        if (p < valid) {
            read_bytes(x + static_cast<uint64_t>(r / x_div) * K, 4ull * K);
            write_bytes(xb + 2ull * p * K, 2ull * K);
        } else {
            write_bytes(y0 + static_cast<uint64_t>(r) * N, 4ull * N);
            if (y1) write_bytes(y1 + static_cast<uint64_t>(r) * N, 4ull * N);
        }
    }
    return launched();
}

hipError_t launch_moe_gemm(const uint8_t *w, float *y, uint32_t routes, uint32_t N, uint32_t K, uint32_t n_experts,
                           uint64_t expert_stride, MoeScratch s, hipStream_t) {
    const uint32_t tiles = s.hdr[1];
    if (tiles > moe_tiles_max(routes, n_experts)) return hipErrorInvalidValue;
    const auto *xb = static_cast<const uint8_t *>(s.x_bf16);
    for (uint32_t t = 0; t < tiles; ++t) {
        const MoeTile tl = s.tiles[t];
        read_bytes(w + tl.expert * expert_stride, static_cast<uint64_t>(N) * row_bytes(K));
        for (uint32_t i = 0; i < tl.count; ++i) {
            const uint32_t p = tl.p0 + i;
            read_bytes(xb + 2ull * p * K, 2ull * K);
            write_bytes(y + static_cast<uint64_t>(s.perm[p]) * N, 4ull * N);
        }
    }
    return launched();
}

}  // namespace q2k
