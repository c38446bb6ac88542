// C ABI of libq2k: argument validation, kernel choice and status reporting.
//
// Every check runs before anything is enqueued, in the validate-then-encode
// order the mlx-native ops use (checked shape products, exact lengths and
// read/write overlap rejection in the op helpers of src/ops/dflash2_selector.rs,
// mlx-native 0.21.1). The per-op rules are those of tests/deepseek_q2_k.rs,
// mlx-native 0.10.8, cited at each entry point in include/q2k.h.
#include "q2k.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "q2k_launch.h"

namespace {

thread_local char g_msg[512];

q2k_status fail(q2k_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return s;
}

q2k_status ok() {
    g_msg[0] = '\0';
    return Q2K_OK;
}

q2k_status device_error(const char *what, hipError_t e) {
    return fail(Q2K_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// a * b with overflow detection.
bool mul_ok(uint64_t a, uint64_t b, uint64_t *out) {
    if (a != 0 && b > UINT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Half-open byte ranges [p, p + n) overlap?
bool overlap(const void *p, uint64_t n, const void *q, uint64_t m) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return n != 0 && m != 0 && a < b + m && b < a + n;
}

struct Range {
    const void *p;
    uint64_t bytes;
};

// Matmul shape rules shared by both kernel choices; also returns byte sizes.
q2k_status check_matmul(const float *x, const void *w, const float *y, uint32_t M, uint32_t N, uint32_t K,
                        Range *rx, Range *rw, Range *ry) {
    if (!x || !w || !y) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: null pointer");
    if (M == 0 || N == 0 || K == 0) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: M, N, K must be >= 1 (got %u, %u, %u)", M, N, K);
    if (K % q2k::kQK != 0) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: K=%u is not a multiple of 256", K);
    if (K > q2k::kMaxK) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: K=%u exceeds the limit %u", K, q2k::kMaxK);
    uint64_t xb, wb, yb, t;
    if (!mul_ok(M, K, &t) || !mul_ok(t, 4, &xb) || !mul_ok(N, K / q2k::kQK, &t) || !mul_ok(t, q2k::kBlockBytes, &wb) ||
        !mul_ok(M, N, &t) || !mul_ok(t, 4, &yb))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: size overflow");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 4))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: x and y must be 16-byte aligned, w 4-byte aligned");
    if (overlap(y, yb, x, xb) || overlap(y, yb, w, wb))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: y overlaps an input");
    *rx = {x, xb};
    *rw = {w, wb};
    *ry = {y, yb};
    return Q2K_OK;
}

// One pinned, device-visible status word per device for the gather's id check.
struct StatusWord {
    int *host = nullptr;
    int *dev = nullptr;
    std::mutex mu;
};

std::mutex g_status_mu;
std::vector<StatusWord *> g_status;  // indexed by device ordinal; never freed

q2k_status status_word(StatusWord **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_error("hipGetDevice", e);
    std::lock_guard<std::mutex> lock(g_status_mu);
    if (g_status.size() <= static_cast<size_t>(dev)) g_status.resize(dev + 1, nullptr);
    if (!g_status[dev]) {
        auto *sw = new StatusWord;
        e = hipHostMalloc(reinterpret_cast<void **>(&sw->host), sizeof(int), hipHostMallocMapped);
        if (e != hipSuccess) {
            delete sw;
            return device_error("hipHostMalloc(status word)", e);
        }
        e = hipHostGetDevicePointer(reinterpret_cast<void **>(&sw->dev), sw->host, 0);
        if (e != hipSuccess) {
            (void)hipHostFree(sw->host);
            delete sw;
            return device_error("hipHostGetDevicePointer(status word)", e);
        }
        g_status[dev] = sw;
    }
    *out = g_status[dev];
    return Q2K_OK;
}

// The matrix-core path (bf16(x)) and the argmax/candidate call (per-chunk
// partials) stage data in a device workspace. One grow-only workspace is kept
// per (device, stream) and used only inside one call; calls on one stream run
// in order, so they can share it. Growth frees and reallocates it in stream
// order, so work already queued on that stream keeps its buffer, and calls on
// different streams never share one.
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

q2k_status stream_workspace(hipStream_t st, size_t bytes, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_error("hipGetDevice", e);
    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace &w = g_ws[{dev, st}];
    if (w.bytes < bytes) {
        if (w.ptr) {
            e = hipFreeAsync(w.ptr, st);
            if (e != hipSuccess) return device_error("hipFreeAsync(workspace)", e);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        e = hipMallocAsync(&w.ptr, bytes, st);
        if (e != hipSuccess) return device_error("hipMallocAsync(workspace)", e);
        w.bytes = bytes;
    }
    *out = w.ptr;
    return Q2K_OK;
}

}  // namespace

namespace q2k {

q2k_status set_error_v(q2k_status s, const char *fmt, va_list ap) {
    std::vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    return s;
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace q2k

extern "C" {

const char *q2k_status_string(q2k_status s) {
    switch (s) {
        case Q2K_OK: return "Q2K_OK";
        case Q2K_ERR_INVALID_ARGUMENT: return "Q2K_ERR_INVALID_ARGUMENT";
        case Q2K_ERR_ID_OUT_OF_RANGE: return "Q2K_ERR_ID_OUT_OF_RANGE";
        case Q2K_ERR_DEVICE: return "Q2K_ERR_DEVICE";
    }
    return "Q2K_UNKNOWN_STATUS";
}

const char *q2k_last_error_message(void) { return g_msg; }

q2k_status q2k_dequantize(const void *blocks, size_t blocks_bytes, float *out, size_t out_elems, void *stream) {
    if (!blocks || !out) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_dequantize: null pointer");
    if (blocks_bytes == 0 || blocks_bytes % q2k::kBlockBytes != 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_dequantize: %zu bytes is not a positive multiple of 84", blocks_bytes);
    const uint64_t nblocks = blocks_bytes / q2k::kBlockBytes;
    uint64_t need, ob;
    if (!mul_ok(nblocks, q2k::kQK, &need) || !mul_ok(out_elems, 4, &ob))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_dequantize: size overflow");
    if (out_elems != need)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_dequantize: %llu blocks need %llu outputs, got %zu",
                    static_cast<unsigned long long>(nblocks), static_cast<unsigned long long>(need), out_elems);
    if (!aligned(blocks, 4) || !aligned(out, 16))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_dequantize: blocks must be 4-byte aligned, out 16-byte aligned");
    if (overlap(out, ob, blocks, blocks_bytes)) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_dequantize: out overlaps blocks");
    hipError_t e = q2k::launch_dequantize(static_cast<const uint8_t *>(blocks), nblocks, out,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_error("q2k_dequantize launch", e);
    return ok();
}

q2k_status q2k_matmul_path(const float *x, const void *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                           q2k_path path, void *stream) {
    Range rx, rw, ry;
    q2k_status s = check_matmul(x, w, y, M, N, K, &rx, &rw, &ry);
    if (s != Q2K_OK) return s;
    if (path == Q2K_PATH_AUTO) path = M <= q2k::kGemvMaxM ? Q2K_PATH_GEMV : Q2K_PATH_MFMA;
    hipError_t e;
    const auto *wb = static_cast<const uint8_t *>(w);
    const auto st = static_cast<hipStream_t>(stream);
    if (path == Q2K_PATH_GEMV) {
        if (M > q2k::kGemvMaxM) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: the GEMV path takes M <= 8 (got %u)", M);
        e = q2k::launch_gemv(x, wb, y, M, N, K, 1, st);
    } else if (path == Q2K_PATH_MFMA) {
        void *ws = nullptr;
        s = stream_workspace(st, static_cast<size_t>(M) * K * 2, &ws);
        if (s != Q2K_OK) return s;
        e = q2k::launch_gemm_mfma(x, wb, y, M, N, K, ws, st);
    } else {
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul: unknown path %d", static_cast<int>(path));
    }
    if (e != hipSuccess) return device_error("q2k_matmul launch", e);
    return ok();
}

q2k_status q2k_matmul(const float *x, const void *w, float *y, uint32_t M, uint32_t N, uint32_t K, void *stream) {
    return q2k_matmul_path(x, w, y, M, N, K, Q2K_PATH_AUTO, stream);
}

q2k_status q2k_matmul_batched(const float *x, const void *w, float *y, uint32_t batches, uint32_t M, uint32_t N,
                              uint32_t K, void *stream) {
    if (!x || !w || !y) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_batched: null pointer");
    if (batches == 0 || M == 0 || N == 0 || K == 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_batched: batches, M, N, K must be >= 1 (got %u, %u, %u, %u)",
                    batches, M, N, K);
    if (M > q2k::kGemvMaxM)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_batched: M=%u; batched mat-vec takes 1 <= M <= 8", M);
    if (K % q2k::kQK != 0) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_batched: K=%u is not a multiple of 256", K);
    if (K > q2k::kMaxK) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_batched: K=%u exceeds the limit %u", K, q2k::kMaxK);
    uint64_t xe, we, ye, t, xb, wbb, yb;
    if (!mul_ok(M, K, &xe) || !mul_ok(N, K / q2k::kQK, &t) || !mul_ok(t, q2k::kBlockBytes, &we) || !mul_ok(M, N, &ye) ||
        !mul_ok(xe, batches, &t) || !mul_ok(t, 4, &xb) || !mul_ok(we, batches, &wbb) || !mul_ok(ye, batches, &t) ||
        !mul_ok(t, 4, &yb))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_batched: size overflow");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 4))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_batched: x and y must be 16-byte aligned, w 4-byte aligned");
    if (overlap(y, yb, x, xb) || overlap(y, yb, w, wbb))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_batched: y overlaps an input");
    const auto st = static_cast<hipStream_t>(stream);
    const auto *wp = static_cast<const uint8_t *>(w);
    for (uint64_t b0 = 0; b0 < batches; b0 += q2k::kMaxGridY) {
        const uint32_t nbat = static_cast<uint32_t>(batches - b0 < q2k::kMaxGridY ? batches - b0 : q2k::kMaxGridY);
        hipError_t e = q2k::launch_gemv(x + b0 * xe, wp + b0 * we, y + b0 * ye, M, N, K, nbat, st);
        if (e != hipSuccess) return device_error("q2k_matmul_batched launch", e);
    }
    return ok();
}

q2k_status q2k_argmax_candidates(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                 uint32_t *top1_idx, float *top1_val, uint32_t *cand_count, uint32_t *overflow,
                                 uint32_t *cand_ids, void *stream) {
    if (!logits || !top1_idx || !top1_val || !cand_count || !overflow || !cand_ids)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_argmax_candidates: null pointer");
    if (n_slots == 0 || vocab == 0 || cap == 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_argmax_candidates: n_slots, vocab, cap must all be > 0 (got %u, %u, %u)",
                    n_slots, vocab, cap);
    if (vocab > q2k::kSampleMaxVocab)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_argmax_candidates: vocab=%u exceeds the limit %u", vocab,
                    q2k::kSampleMaxVocab);
    uint64_t lb, cb, t;
    if (!mul_ok(n_slots, vocab, &t) || !mul_ok(t, 4, &lb) || !mul_ok(n_slots, cap, &t) || !mul_ok(t, 4, &cb))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_argmax_candidates: size overflow");
    if (!aligned(logits, 4) || !aligned(top1_idx, 4) || !aligned(top1_val, 4) || !aligned(cand_count, 4) ||
        !aligned(overflow, 4) || !aligned(cand_ids, 4))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_argmax_candidates: every buffer must be 4-byte aligned");
    const Range outs[5] = {{top1_idx, 4ull * n_slots}, {top1_val, 4ull * n_slots}, {cand_count, 4ull * n_slots},
                           {overflow, 4ull * n_slots}, {cand_ids, cb}};
    for (int i = 0; i < 5; ++i) {
        if (overlap(outs[i].p, outs[i].bytes, logits, lb))
            return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_argmax_candidates: an output overlaps the logits");
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
                return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_argmax_candidates: outputs overlap each other");
    }
    const auto st = static_cast<hipStream_t>(stream);
    for (uint64_t s0 = 0; s0 < n_slots; s0 += q2k::kMaxGridY) {
        const uint32_t ns = static_cast<uint32_t>(n_slots - s0 < q2k::kMaxGridY ? n_slots - s0 : q2k::kMaxGridY);
        void *ws = nullptr;
        q2k_status s = stream_workspace(st, q2k::sample_workspace_bytes(ns, vocab), &ws);
        if (s != Q2K_OK) return s;
        hipError_t e = q2k::launch_argmax_candidates(logits + s0 * vocab, ns, vocab, cap, top1_idx + s0, top1_val + s0,
                                                     cand_count + s0, overflow + s0, cand_ids + s0 * cap, ws, st);
        if (e != hipSuccess) return device_error("q2k_argmax_candidates launch", e);
    }
    return ok();
}

q2k_status q2k_embedding_gather(const void *table, const uint32_t *ids, float *out, uint32_t vocab,
                                uint32_t embed_dim, uint32_t n_tokens, void *stream) {
    if (!table || !ids || !out) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather: null pointer");
    if (vocab == 0 || embed_dim == 0 || n_tokens == 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather: vocab, embed_dim, n_tokens must be >= 1 (got %u, %u, %u)",
                    vocab, embed_dim, n_tokens);
    if (embed_dim % q2k::kQK != 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather: embed_dim=%u is not a multiple of 256", embed_dim);
    const uint32_t bpr = embed_dim / q2k::kQK;
    uint64_t tb, ob, ib, t;
    if (!mul_ok(vocab, bpr, &t) || !mul_ok(t, q2k::kBlockBytes, &tb) || !mul_ok(n_tokens, embed_dim, &t) ||
        !mul_ok(t, 4, &ob) || !mul_ok(n_tokens, 4, &ib))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather: size overflow");
    if (!aligned(table, 4) || !aligned(ids, 4) || !aligned(out, 16))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather: table and ids must be 4-byte aligned, out 16-byte aligned");
    if (overlap(out, ob, table, tb) || overlap(out, ob, ids, ib))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather: out overlaps an input");

    StatusWord *sw = nullptr;
    q2k_status s = status_word(&sw);
    if (s != Q2K_OK) return s;
    std::lock_guard<std::mutex> lock(sw->mu);
    *sw->host = 0;
    const auto st = static_cast<hipStream_t>(stream);
    hipError_t e = q2k::launch_gather(static_cast<const uint8_t *>(table), ids, out, vocab, bpr, n_tokens, sw->dev, st);
    if (e != hipSuccess) return device_error("q2k_embedding_gather launch", e);
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return device_error("q2k_embedding_gather sync", e);
    const int bad = __atomic_load_n(sw->host, __ATOMIC_ACQUIRE);
    if (bad) return fail(Q2K_ERR_ID_OUT_OF_RANGE, "q2k_embedding_gather: a token id is >= vocab (%u)", vocab);
    return ok();
}

}  // extern "C"
