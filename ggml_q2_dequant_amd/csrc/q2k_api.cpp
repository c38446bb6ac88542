// C ABI of libq2k: argument validation, kernel choice and status reporting.
//
// Every check runs before anything is enqueued, in the validate-then-encode
// order the mlx-native ops use (checked shape products, exact lengths and
// read/write overlap rejection in the op helpers of src/ops/dflash2_selector.rs,
// mlx-native 0.21.1). The per-op rules are those of tests/deepseek_q2_k.rs,
// mlx-native 0.10.8, cited at each entry point in include/q2k.h.
#include "q2k.h"

#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <memory>
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

// Per device, for the synchronous gather: a device word the gather kernel
// stores a bad id's marker into, and a pinned, host-coherent word that a
// one-thread kernel queued behind it publishes the outcome to. The host polls
// the pinned word instead of synchronizing the stream, which costs several
// microseconds more per call. Each call tags its marker and its published
// word with a fresh sequence number, so nothing an earlier call left behind
// reads as this call's; the completion kernel also clears the device word. A
// call that launched the gather but not its completion kernel marks the word
// for clearing before the next call.
struct StatusWord {
    int *host = nullptr;      // pinned, mapped, coherent
    int *host_dev = nullptr;  // the same word's device address
    int *dev = nullptr;       // device memory, zero between calls
    uint32_t seq = 0;
    bool stale = false;
    std::mutex mu;
};

std::mutex g_status_mu;
// Indexed by device ordinal. Neither the vector nor its words are ever freed,
// so a call made while the process exits still finds them.
std::vector<StatusWord *> &g_status = *new std::vector<StatusWord *>;

// Argument rules shared by both gather entry points (sizes, alignment, overlap).
q2k_status check_gather(const char *fn, const void *table, const uint32_t *ids, float *out, uint32_t vocab,
                        uint32_t embed_dim, uint32_t n_tokens) {
    if (!table || !ids || !out) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (vocab == 0 || embed_dim == 0 || n_tokens == 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: vocab, embed_dim, n_tokens must be >= 1 (got %u, %u, %u)", fn,
                    vocab, embed_dim, n_tokens);
    if (embed_dim % q2k::kQK != 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: embed_dim=%u is not a multiple of 256", fn, embed_dim);
    const uint32_t bpr = embed_dim / q2k::kQK;
    uint64_t tb, ob, ib, t;
    if (!mul_ok(vocab, bpr, &t) || !mul_ok(t, q2k::kBlockBytes, &tb) || !mul_ok(n_tokens, embed_dim, &t) ||
        !mul_ok(t, 4, &ob) || !mul_ok(n_tokens, 4, &ib))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: size overflow", fn);
    if (!aligned(table, 4) || !aligned(ids, 4) || !aligned(out, 16))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: table and ids must be 4-byte aligned, out 16-byte aligned", fn);
    if (overlap(out, ob, table, tb) || overlap(out, ob, ids, ib))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: out overlaps an input", fn);
    return Q2K_OK;
}

q2k_status status_word(StatusWord **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_error("hipGetDevice", e);
    std::lock_guard<std::mutex> lock(g_status_mu);
    if (g_status.size() <= static_cast<size_t>(dev)) g_status.resize(dev + 1, nullptr);
    if (!g_status[dev]) {
        auto *sw = new StatusWord;
        e = hipHostMalloc(reinterpret_cast<void **>(&sw->host), sizeof(int), hipHostMallocMapped | hipHostMallocCoherent);
        if (e != hipSuccess) {
            delete sw;
            return device_error("hipHostMalloc(status word)", e);
        }
        *sw->host = 0;
        e = hipHostGetDevicePointer(reinterpret_cast<void **>(&sw->host_dev), sw->host, 0);
        if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&sw->dev), sizeof(int));
        if (e == hipSuccess) e = hipMemset(sw->dev, 0, sizeof(int));
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            if (sw->dev) (void)hipFree(sw->dev);
            (void)hipHostFree(sw->host);
            delete sw;
            return device_error("status word set-up", e);
        }
        g_status[dev] = sw;
    }
    *out = g_status[dev];
    return Q2K_OK;
}

// The matrix-core path (bf16(x)), the matrix-core expert-routed schedule
// (routing tables and bf16 rows) and the argmax/candidate call (per-chunk
// partials) stage data in device scratch. The *_pooled entry points take it
// from the caller; the others use a workspace libq2k keeps per (device,
// stream):
//  - a call holds that workspace's lock from its size check until its
//    launches are enqueued, so a call from another host thread on the same
//    stream cannot replace the buffer between the two;
//  - the workspace only grows, and a buffer that a larger request replaces is
//    never freed: a HIP graph captured earlier may still hold its address.
//    Retired buffers stay allocated until the process ends; growth at least
//    doubles the size, so together they never exceed the live buffer;
//  - growth is refused while the stream is capturing a graph (the allocation
//    would not be part of the graph's own memory): one eager call of the
//    largest size first, or the pooled form, avoids it.
struct Workspace {
    std::mutex mu;
    void *ptr = nullptr;
    size_t bytes = 0;
    std::vector<void *> retired;
};

std::mutex g_ws_mu;  // guards the map, not the workspaces
// Never destroyed (like the buffers it holds), so a call made while the
// process exits still finds it.
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Workspace>> &g_ws =
    *new std::map<std::pair<int, hipStream_t>, std::unique_ptr<Workspace>>;

// Calls launch(buffer) with the stream's workspace grown to at least `bytes`,
// holding the workspace's lock until launch returns. launch returns a status.
template <class F>
q2k_status with_workspace(const char *fn, hipStream_t st, size_t bytes, F &&launch) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_error("hipGetDevice", e);
    Workspace *w;
    {
        std::lock_guard<std::mutex> lock(g_ws_mu);
        std::unique_ptr<Workspace> &slot = g_ws[{dev, st}];
        if (!slot) slot.reset(new Workspace);
        w = slot.get();
    }
    std::lock_guard<std::mutex> lock(w->mu);
    if (w->bytes < bytes) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(st, &cs);
        if (e != hipSuccess) return device_error("hipStreamIsCapturing", e);
        if (cs != hipStreamCaptureStatusNone)
            return fail(Q2K_ERR_INVALID_ARGUMENT,
                        "%s: the stream's workspace must grow to %zu bytes, which is not done during graph capture; "
                        "make one call of this size before capturing, or pass scratch to the pooled form",
                        fn, bytes);
        const size_t want = bytes > 2 * w->bytes ? bytes : 2 * w->bytes;
        void *p = nullptr;
        e = hipMalloc(&p, want);
        if (e != hipSuccess) return device_error("hipMalloc(workspace)", e);
        if (w->ptr) w->retired.push_back(w->ptr);
        w->ptr = p;
        w->bytes = want;
    }
    return launch(w->ptr);
}

// Caller scratch: non-null, 256-byte aligned, at least `need` bytes, and
// disjoint from every other argument.
q2k_status check_caller_scratch(const char *fn, const void *scratch, uint64_t scratch_bytes, uint64_t need,
                                const Range *args, int n_args) {
    if (!scratch) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: null scratch", fn);
    if (!aligned(scratch, 256)) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: scratch must be 256-byte aligned", fn);
    if (scratch_bytes < need)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: scratch holds %llu bytes, %llu needed", fn,
                    static_cast<unsigned long long>(scratch_bytes), static_cast<unsigned long long>(need));
    for (int i = 0; i < n_args; ++i)
        if (overlap(scratch, need, args[i].p, args[i].bytes))
            return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: scratch overlaps another argument", fn);
    return Q2K_OK;
}

// Shape rules of the expert-routed calls; sizes in bytes of x, w, ids, y.
struct MoeShape {
    uint32_t routes, x_div;
    Range x, w, ids, y;
};

q2k_status check_moe_shape(const char *fn, const q2k_matmul_id_params *p, bool slotted, MoeShape *out) {
    if (!p) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (p->reserved != 0) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: params.reserved must be 0", fn);
    if (p->n_tokens == 0 || p->top_k == 0 || p->n == 0 || p->k == 0 || p->n_experts == 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: n_tokens, top_k, n, k, n_experts must be >= 1 (got %u, %u, %u, %u, %u)",
                    fn, p->n_tokens, p->top_k, p->n, p->k, p->n_experts);
    if (p->k % q2k::kQK != 0) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: k=%u is not a multiple of 256", fn, p->k);
    if (p->k > q2k::kMaxK) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: k=%u exceeds the limit %u", fn, p->k, q2k::kMaxK);
    if (p->n_experts > q2k::kMoeMaxExperts)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: n_experts=%u exceeds the limit %u", fn, p->n_experts,
                    q2k::kMoeMaxExperts);
    uint64_t routes, t, rb, xb, wb, yb;
    if (!mul_ok(p->n_tokens, p->top_k, &routes) || routes > q2k::kMoeMaxRoutes)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: n_tokens * top_k exceeds the limit %u", fn, q2k::kMoeMaxRoutes);
    rb = static_cast<uint64_t>(p->k / q2k::kQK) * q2k::kBlockBytes;
    uint64_t expert_bytes;
    if (!mul_ok(p->n, rb, &expert_bytes)) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: size overflow", fn);
    if (p->expert_stride < expert_bytes || p->expert_stride % 4 != 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: expert_stride=%llu must be a multiple of 4 and >= n * k/256 * 84 = %llu",
                    fn, static_cast<unsigned long long>(p->expert_stride), static_cast<unsigned long long>(expert_bytes));
    if (!mul_ok(p->n_experts - 1, p->expert_stride, &t) || t > UINT64_MAX - expert_bytes)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: size overflow", fn);
    wb = t + expert_bytes;
    if (!mul_ok(slotted ? routes : p->n_tokens, p->k, &t) || !mul_ok(t, 4, &xb) || !mul_ok(routes, p->n, &t) ||
        !mul_ok(t, 4, &yb))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: size overflow", fn);
    out->routes = static_cast<uint32_t>(routes);
    out->x_div = slotted ? 1u : p->top_k;
    out->x = {nullptr, xb};
    out->w = {nullptr, wb};
    out->ids = {nullptr, 4 * routes};
    out->y = {nullptr, yb};
    return Q2K_OK;
}

q2k_status check_moe(const char *fn, const float *x, const void *w, const uint32_t *ids, const float *y,
                     const q2k_matmul_id_params *p, bool slotted, MoeShape *out) {
    if (!x || !w || !ids || !y || !p) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    q2k_status s = check_moe_shape(fn, p, slotted, out);
    if (s != Q2K_OK) return s;
    const uint64_t xb = out->x.bytes, wb = out->w.bytes, yb = out->y.bytes, routes = out->routes;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 4) || !aligned(ids, 4))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: x and y must be 16-byte aligned, w and ids 4-byte aligned", fn);
    if (overlap(y, yb, x, xb) || overlap(y, yb, w, wb) || overlap(y, yb, ids, 4 * routes))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: y overlaps an input", fn);
    out->x = {x, xb};
    out->w = {w, wb};
    out->ids = {ids, 4 * routes};
    out->y = {y, yb};
    return Q2K_OK;
}

q2k_status check_status_word(const char *fn, const int *status, const Range *outs, int n_outs) {
    if (!status) return Q2K_OK;
    if (!aligned(status, 4)) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: status must be 4-byte aligned", fn);
    for (int i = 0; i < n_outs; ++i)
        if (overlap(status, 4, outs[i].p, outs[i].bytes))
            return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: status overlaps another argument", fn);
    return Q2K_OK;
}

// The matrix-core schedule: route, gather, then one GEMM per weight set.
q2k_status run_moe_mfma(const char *fn, const MoeShape &sh, const q2k_matmul_id_params *p, const void *w0,
                        const void *w1, float *y0, float *y1, void *scratch, int *status, hipStream_t st) {
    const q2k::MoeScratch sc = q2k::moe_scratch_carve(scratch, sh.routes, p->n_experts);
    hipError_t e = q2k::launch_moe_route(static_cast<const uint32_t *>(sh.ids.p), sh.routes, p->n_experts, sc, status, st);
    if (e == hipSuccess)
        e = q2k::launch_moe_gather(static_cast<const float *>(sh.x.p), sh.routes, sh.x_div, p->k, sc, y0, y1, p->n, st);
    if (e == hipSuccess)
        e = q2k::launch_moe_gemm(static_cast<const uint8_t *>(w0), y0, sh.routes, p->n, p->k, p->n_experts,
                                 p->expert_stride, sc, st);
    if (e == hipSuccess && w1)
        e = q2k::launch_moe_gemm(static_cast<const uint8_t *>(w1), y1, sh.routes, p->n, p->k, p->n_experts,
                                 p->expert_stride, sc, st);
    if (e != hipSuccess) return device_error(fn, e);
    return ok();
}

q2k_status check_scratch(const char *fn, const MoeShape &sh, const q2k_matmul_id_params *p, const void *scratch,
                         uint64_t scratch_bytes, const Range *args, int n_args) {
    return check_caller_scratch(fn, scratch, scratch_bytes, q2k::moe_scratch_bytes(sh.routes, p->n_experts, p->k), args,
                                n_args);
}

// Kernel choice of a matmul call: Q2K_PATH_AUTO resolves to the fp32 GEMV for
// M <= 8 and to the matrix cores above; the GEMV takes M <= 8 only.
q2k_status resolve_path(const char *fn, uint32_t M, q2k_path *path) {
    if (*path == Q2K_PATH_AUTO) *path = M <= q2k::kGemvMaxM ? Q2K_PATH_GEMV : Q2K_PATH_MFMA;
    if (*path == Q2K_PATH_GEMV && M > q2k::kGemvMaxM)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: the GEMV path takes M <= 8 (got %u)", fn, M);
    if (*path != Q2K_PATH_GEMV && *path != Q2K_PATH_MFMA)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: unknown path %d", fn, static_cast<int>(*path));
    return Q2K_OK;
}

// Scratch bytes of a resolved matmul path: bf16(x) for the matrix cores.
uint64_t matmul_scratch(uint32_t M, uint32_t K, q2k_path path) {
    return path == Q2K_PATH_MFMA ? 2ull * M * K : 0;
}

// Enqueues a validated matmul; scratch (for the matrix-core path) is caller
// memory, or null for the stream's workspace.
q2k_status run_matmul(const char *fn, const float *x, const uint8_t *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                      q2k_path path, void *scratch, hipStream_t st) {
    hipError_t e;
    if (path == Q2K_PATH_GEMV) {
        e = q2k::launch_gemv(x, w, y, M, N, K, 1, st);
    } else if (scratch) {
        e = q2k::launch_gemm_mfma(x, w, y, M, N, K, scratch, st);
    } else {
        e = hipSuccess;
        const q2k_status s = with_workspace(fn, st, matmul_scratch(M, K, path), [&](void *ws) {
            e = q2k::launch_gemm_mfma(x, w, y, M, N, K, ws, st);
            return Q2K_OK;
        });
        if (s != Q2K_OK) return s;
    }
    if (e != hipSuccess) return device_error(fn, e);
    return ok();
}

// Argument rules of the argmax/candidate calls.
q2k_status check_argmax(const char *fn, const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                        const uint32_t *top1_idx, const float *top1_val, const uint32_t *cand_count,
                        const uint32_t *overflow, const uint32_t *cand_ids, Range *args) {
    if (!logits || !top1_idx || !top1_val || !cand_count || !overflow || !cand_ids)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (n_slots == 0 || vocab == 0 || cap == 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: n_slots, vocab, cap must all be > 0 (got %u, %u, %u)", fn, n_slots,
                    vocab, cap);
    if (vocab > q2k::kSampleMaxVocab)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: vocab=%u exceeds the limit %u", fn, vocab, q2k::kSampleMaxVocab);
    uint64_t lb, cb, t;
    if (!mul_ok(n_slots, vocab, &t) || !mul_ok(t, 4, &lb) || !mul_ok(n_slots, cap, &t) || !mul_ok(t, 4, &cb))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: size overflow", fn);
    if (!aligned(logits, 4) || !aligned(top1_idx, 4) || !aligned(top1_val, 4) || !aligned(cand_count, 4) ||
        !aligned(overflow, 4) || !aligned(cand_ids, 4))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: every buffer must be 4-byte aligned", fn);
    const Range outs[5] = {{top1_idx, 4ull * n_slots}, {top1_val, 4ull * n_slots}, {cand_count, 4ull * n_slots},
                           {overflow, 4ull * n_slots}, {cand_ids, cb}};
    for (int i = 0; i < 5; ++i) {
        if (overlap(outs[i].p, outs[i].bytes, logits, lb))
            return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: an output overlaps the logits", fn);
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
                return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: outputs overlap each other", fn);
    }
    args[0] = {logits, lb};
    for (int i = 0; i < 5; ++i) args[1 + i] = outs[i];
    return Q2K_OK;
}

// Scratch of the argmax/candidate call: the per-chunk partials of the largest
// launch (at most kMaxGridY slots; later launches of a call reuse it in order).
uint64_t argmax_scratch(uint32_t n_slots, uint32_t vocab) {
    return q2k::sample_workspace_bytes(n_slots < q2k::kMaxGridY ? n_slots : q2k::kMaxGridY, vocab);
}

hipError_t run_argmax(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap, uint32_t *top1_idx,
                      float *top1_val, uint32_t *cand_count, uint32_t *overflow, uint32_t *cand_ids, void *ws,
                      hipStream_t st) {
    for (uint64_t s0 = 0; s0 < n_slots; s0 += q2k::kMaxGridY) {
        const uint32_t ns = static_cast<uint32_t>(n_slots - s0 < q2k::kMaxGridY ? n_slots - s0 : q2k::kMaxGridY);
        const hipError_t e = q2k::launch_argmax_candidates(logits + s0 * vocab, ns, vocab, cap, top1_idx + s0,
                                                           top1_val + s0, cand_count + s0, overflow + s0,
                                                           cand_ids + s0 * cap, ws, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
    if ((s = resolve_path("q2k_matmul", M, &path)) != Q2K_OK) return s;
    return run_matmul("q2k_matmul", x, static_cast<const uint8_t *>(w), y, M, N, K, path, nullptr,
                      static_cast<hipStream_t>(stream));
}

q2k_status q2k_matmul_scratch_bytes(uint32_t M, uint32_t N, uint32_t K, q2k_path path, uint64_t *bytes) {
    if (!bytes) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_scratch_bytes: null pointer");
    if (M == 0 || N == 0 || K == 0)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_scratch_bytes: M, N, K must be >= 1 (got %u, %u, %u)", M, N, K);
    if (K % q2k::kQK != 0 || K > q2k::kMaxK)
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_matmul_scratch_bytes: K=%u is not a multiple of 256 in 256..%u", K,
                    q2k::kMaxK);
    q2k_status s = resolve_path("q2k_matmul_scratch_bytes", M, &path);
    if (s != Q2K_OK) return s;
    *bytes = matmul_scratch(M, K, path);
    return ok();
}

q2k_status q2k_matmul_pooled(const float *x, const void *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                             q2k_path path, void *scratch, uint64_t scratch_bytes, void *stream) {
    static const char fn[] = "q2k_matmul_pooled";
    Range rx, rw, ry;
    q2k_status s = check_matmul(x, w, y, M, N, K, &rx, &rw, &ry);
    if (s != Q2K_OK) return s;
    if ((s = resolve_path(fn, M, &path)) != Q2K_OK) return s;
    const uint64_t need = matmul_scratch(M, K, path);
    if (need == 0) {
        scratch = nullptr;
    } else {
        const Range args[3] = {rx, rw, ry};
        if ((s = check_caller_scratch(fn, scratch, scratch_bytes, need, args, 3)) != Q2K_OK) return s;
    }
    return run_matmul(fn, x, static_cast<const uint8_t *>(w), y, M, N, K, path, scratch,
                      static_cast<hipStream_t>(stream));
}

q2k_status q2k_matmul_noalloc(const float *x, const void *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                              void *stream) {
    static const char fn[] = "q2k_matmul_noalloc";
    Range rx, rw, ry;
    q2k_status s = check_matmul(x, w, y, M, N, K, &rx, &rw, &ry);
    if (s != Q2K_OK) return s;
    q2k_path path = Q2K_PATH_AUTO;
    if ((s = resolve_path(fn, M, &path)) != Q2K_OK) return s;
    const uint64_t need = matmul_scratch(M, K, path);
    void *scratch = nullptr;
    if (need > 0) {
        if (need > q2k::kNoAllocScratchBytes)
            return fail(Q2K_ERR_INVALID_ARGUMENT,
                        "%s: M=%u, K=%u needs %llu bytes of bf16 activations; the library's device scratch holds "
                        "%llu (M * K <= %llu when M > 8)",
                        fn, M, K, static_cast<unsigned long long>(need),
                        static_cast<unsigned long long>(q2k::kNoAllocScratchBytes),
                        static_cast<unsigned long long>(q2k::kNoAllocScratchBytes / 2));
        const hipError_t e = q2k::noalloc_scratch(&scratch);
        if (e != hipSuccess) return device_error("q2k_matmul_noalloc: hipGetSymbolAddress(scratch)", e);
    }
    return run_matmul(fn, x, static_cast<const uint8_t *>(w), y, M, N, K, path, scratch,
                      static_cast<hipStream_t>(stream));
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
    // Problems per launch: at most kMaxGridY.
    const uint64_t per = q2k::kMaxGridY;
    for (uint64_t b0 = 0; b0 < batches; b0 += per) {
        const uint32_t nbat = static_cast<uint32_t>(batches - b0 < per ? batches - b0 : per);
        hipError_t e = q2k::launch_gemv(x + b0 * xe, wp + b0 * we, y + b0 * ye, M, N, K, nbat, st);
        if (e != hipSuccess) return device_error("q2k_matmul_batched launch", e);
    }
    return ok();
}

q2k_status q2k_argmax_candidates(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                 uint32_t *top1_idx, float *top1_val, uint32_t *cand_count, uint32_t *overflow,
                                 uint32_t *cand_ids, void *stream) {
    static const char fn[] = "q2k_argmax_candidates";
    Range args[6];
    q2k_status s = check_argmax(fn, logits, n_slots, vocab, cap, top1_idx, top1_val, cand_count, overflow, cand_ids,
                                args);
    if (s != Q2K_OK) return s;
    const auto st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    s = with_workspace(fn, st, argmax_scratch(n_slots, vocab), [&](void *ws) {
        e = run_argmax(logits, n_slots, vocab, cap, top1_idx, top1_val, cand_count, overflow, cand_ids, ws, st);
        return Q2K_OK;
    });
    if (s != Q2K_OK) return s;
    if (e != hipSuccess) return device_error(fn, e);
    return ok();
}

q2k_status q2k_argmax_candidates_scratch_bytes(uint32_t n_slots, uint32_t vocab, uint64_t *bytes) {
    if (!bytes) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_argmax_candidates_scratch_bytes: null pointer");
    if (n_slots == 0 || vocab == 0 || vocab > q2k::kSampleMaxVocab)
        return fail(Q2K_ERR_INVALID_ARGUMENT,
                    "q2k_argmax_candidates_scratch_bytes: need n_slots >= 1 and 1 <= vocab <= %u (got %u, %u)",
                    q2k::kSampleMaxVocab, n_slots, vocab);
    *bytes = argmax_scratch(n_slots, vocab);
    return ok();
}

q2k_status q2k_argmax_candidates_pooled(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                        uint32_t *top1_idx, float *top1_val, uint32_t *cand_count, uint32_t *overflow,
                                        uint32_t *cand_ids, void *scratch, uint64_t scratch_bytes, void *stream) {
    static const char fn[] = "q2k_argmax_candidates_pooled";
    Range args[6];
    q2k_status s = check_argmax(fn, logits, n_slots, vocab, cap, top1_idx, top1_val, cand_count, overflow, cand_ids,
                                args);
    if (s != Q2K_OK) return s;
    if ((s = check_caller_scratch(fn, scratch, scratch_bytes, argmax_scratch(n_slots, vocab), args, 6)) != Q2K_OK)
        return s;
    const hipError_t e = run_argmax(logits, n_slots, vocab, cap, top1_idx, top1_val, cand_count, overflow, cand_ids,
                                    scratch, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_error(fn, e);
    return ok();
}

q2k_status q2k_matmul_id_path(const float *x, const void *w, const uint32_t *ids, float *y,
                              const q2k_matmul_id_params *p, int *status, q2k_path path, void *stream) {
    static const char fn[] = "q2k_matmul_id";
    MoeShape sh;
    q2k_status s = check_moe(fn, x, w, ids, y, p, false, &sh);
    if (s != Q2K_OK) return s;
    const Range args[4] = {sh.x, sh.w, sh.ids, sh.y};
    if ((s = check_status_word(fn, status, args, 4)) != Q2K_OK) return s;
    if (path == Q2K_PATH_AUTO)
        path = p->n_tokens > 32 && (p->top_k == 1 || p->top_k == 6 || p->top_k == 8) ? Q2K_PATH_MFMA : Q2K_PATH_GEMV;
    const auto st = static_cast<hipStream_t>(stream);
    if (path == Q2K_PATH_GEMV) {
        hipError_t e = q2k::launch_moe_gemv(x, static_cast<const uint8_t *>(w), ids, y, sh.routes, sh.x_div, p->n, p->k,
                                            p->n_experts, p->expert_stride, status, st);
        if (e != hipSuccess) return device_error(fn, e);
        return ok();
    }
    if (path != Q2K_PATH_MFMA) return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: unknown path %d", fn, static_cast<int>(path));
    return with_workspace(fn, st, q2k::moe_scratch_bytes(sh.routes, p->n_experts, p->k), [&](void *ws) {
        return run_moe_mfma(fn, sh, p, w, nullptr, y, nullptr, ws, status, st);
    });
}

q2k_status q2k_matmul_id(const float *x, const void *w, const uint32_t *ids, float *y,
                         const q2k_matmul_id_params *p, int *status, void *stream) {
    return q2k_matmul_id_path(x, w, ids, y, p, status, Q2K_PATH_AUTO, stream);
}

uint64_t q2k_matmul_id_scratch_bytes(const q2k_matmul_id_params *p) {
    MoeShape sh;
    if (check_moe_shape("q2k_matmul_id_scratch_bytes", p, false, &sh) != Q2K_OK) return 0;
    return q2k::moe_scratch_bytes(sh.routes, p->n_experts, p->k);
}

q2k_status q2k_matmul_id_pooled(const float *x, const void *w, const uint32_t *ids, float *y,
                                const q2k_matmul_id_params *p, void *scratch, uint64_t scratch_bytes, int *status,
                                void *stream) {
    static const char fn[] = "q2k_matmul_id_pooled";
    MoeShape sh;
    q2k_status s = check_moe(fn, x, w, ids, y, p, false, &sh);
    if (s != Q2K_OK) return s;
    const Range args[4] = {sh.x, sh.w, sh.ids, sh.y};
    if ((s = check_scratch(fn, sh, p, scratch, scratch_bytes, args, 4)) != Q2K_OK) return s;
    const Range args2[5] = {sh.x, sh.w, sh.ids, sh.y, {scratch, scratch_bytes}};
    if ((s = check_status_word(fn, status, args2, 5)) != Q2K_OK) return s;
    return run_moe_mfma(fn, sh, p, w, nullptr, y, nullptr, scratch, status, static_cast<hipStream_t>(stream));
}

q2k_status q2k_matmul_id_pooled_pair(const float *x, const void *w0, const void *w1, const uint32_t *ids, float *y0,
                                     float *y1, const q2k_matmul_id_params *p, void *scratch, uint64_t scratch_bytes,
                                     int *status, void *stream) {
    static const char fn[] = "q2k_matmul_id_pooled_pair";
    MoeShape s0, s1;
    q2k_status s = check_moe(fn, x, w0, ids, y0, p, false, &s0);
    if (s != Q2K_OK) return s;
    if ((s = check_moe(fn, x, w1, ids, y1, p, false, &s1)) != Q2K_OK) return s;
    if (overlap(y0, s0.y.bytes, y1, s1.y.bytes) || overlap(y0, s0.y.bytes, w1, s1.w.bytes) ||
        overlap(y1, s1.y.bytes, w0, s0.w.bytes))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "%s: an output overlaps the other output or weight set", fn);
    const Range args[6] = {s0.x, s0.w, s1.w, s0.ids, s0.y, s1.y};
    if ((s = check_scratch(fn, s0, p, scratch, scratch_bytes, args, 6)) != Q2K_OK) return s;
    const Range args2[7] = {s0.x, s0.w, s1.w, s0.ids, s0.y, s1.y, {scratch, scratch_bytes}};
    if ((s = check_status_word(fn, status, args2, 7)) != Q2K_OK) return s;
    return run_moe_mfma(fn, s0, p, w0, w1, y0, y1, scratch, status, static_cast<hipStream_t>(stream));
}

q2k_status q2k_matmul_id_pooled_slotted(const float *x, const void *w, const uint32_t *ids, float *y,
                                        const q2k_matmul_id_params *p, void *scratch, uint64_t scratch_bytes,
                                        int *status, void *stream) {
    static const char fn[] = "q2k_matmul_id_pooled_slotted";
    MoeShape sh;
    q2k_status s = check_moe(fn, x, w, ids, y, p, true, &sh);
    if (s != Q2K_OK) return s;
    const Range args[4] = {sh.x, sh.w, sh.ids, sh.y};
    if ((s = check_scratch(fn, sh, p, scratch, scratch_bytes, args, 4)) != Q2K_OK) return s;
    const Range args2[5] = {sh.x, sh.w, sh.ids, sh.y, {scratch, scratch_bytes}};
    if ((s = check_status_word(fn, status, args2, 5)) != Q2K_OK) return s;
    return run_moe_mfma(fn, sh, p, w, nullptr, y, nullptr, scratch, status, static_cast<hipStream_t>(stream));
}

q2k_status q2k_embedding_gather(const void *table, const uint32_t *ids, float *out, uint32_t vocab,
                                uint32_t embed_dim, uint32_t n_tokens, void *stream) {
    q2k_status s = check_gather("q2k_embedding_gather", table, ids, out, vocab, embed_dim, n_tokens);
    if (s != Q2K_OK) return s;
    const auto st = static_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess) return device_error("hipStreamIsCapturing", e);
    if (cs != hipStreamCaptureStatusNone)
        return fail(Q2K_ERR_INVALID_ARGUMENT,
                    "q2k_embedding_gather: waits on the host, so it cannot be captured; use q2k_embedding_gather_async");
    StatusWord *sw = nullptr;
    s = status_word(&sw);
    if (s != Q2K_OK) return s;
    std::lock_guard<std::mutex> lock(sw->mu);
    if (sw->stale) {
        // A gather launched by the failed call may still be running (on any stream): let it end first.
        e = hipDeviceSynchronize();
        if (e == hipSuccess) e = hipMemset(sw->dev, 0, sizeof(int));
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) return device_error("q2k_embedding_gather: status word reset", e);
        sw->stale = false;
    }
    // Sequence numbers run over 1 .. 2^29 - 1, so (seq << 2) | 3 stays a positive int.
    sw->seq = sw->seq % ((1u << 29) - 1) + 1;
    const int seq = static_cast<int>(sw->seq);
    e = q2k::launch_gather(static_cast<const uint8_t *>(table), ids, out, vocab, embed_dim / q2k::kQK, n_tokens,
                           sw->dev, seq, st);
    if (e != hipSuccess) return device_error("q2k_embedding_gather launch", e);
    e = q2k::launch_gather_done(sw->dev, seq, sw->host_dev, st);
    if (e != hipSuccess) {
        sw->stale = true;
        return device_error("q2k_embedding_gather launch", e);
    }
    // Poll for the published word; past about 2 ms (a stream with other work
    // queued ahead) wait on the stream instead, which also reports any fault.
    const int want = (seq << 2) | 2;
    int v = __atomic_load_n(sw->host, __ATOMIC_ACQUIRE);
    if ((v & ~1) != want) {
        const auto t0 = std::chrono::steady_clock::now();
        for (;;) {
            v = __atomic_load_n(sw->host, __ATOMIC_ACQUIRE);
            if ((v & ~1) == want) break;
            if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(2)) {
                e = hipStreamSynchronize(st);
                if (e != hipSuccess) return device_error("q2k_embedding_gather sync", e);
                v = __atomic_load_n(sw->host, __ATOMIC_ACQUIRE);
                if ((v & ~1) != want) {
                    sw->stale = true;
                    return fail(Q2K_ERR_DEVICE, "q2k_embedding_gather: the completion word was not published");
                }
                break;
            }
        }
    }
    if (v & 1) return fail(Q2K_ERR_ID_OUT_OF_RANGE, "q2k_embedding_gather: a token id is >= vocab (%u)", vocab);
    return ok();
}

q2k_status q2k_embedding_gather_async(const void *table, const uint32_t *ids, float *out, uint32_t vocab,
                                      uint32_t embed_dim, uint32_t n_tokens, int *status, void *stream) {
    q2k_status s = check_gather("q2k_embedding_gather_async", table, ids, out, vocab, embed_dim, n_tokens);
    if (s != Q2K_OK) return s;
    if (!status) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather_async: status is required");
    if (!aligned(status, 4)) return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather_async: status must be 4-byte aligned");
    const uint64_t ob = static_cast<uint64_t>(n_tokens) * embed_dim * 4;
    const uint64_t tb = static_cast<uint64_t>(vocab) * (embed_dim / q2k::kQK) * q2k::kBlockBytes;
    if (overlap(status, 4, out, ob) || overlap(status, 4, table, tb) || overlap(status, 4, ids, 4ull * n_tokens))
        return fail(Q2K_ERR_INVALID_ARGUMENT, "q2k_embedding_gather_async: status overlaps an input or out");
    hipError_t e = q2k::launch_gather(static_cast<const uint8_t *>(table), ids, out, vocab, embed_dim / q2k::kQK,
                                      n_tokens, status, 1, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_error("q2k_embedding_gather_async launch", e);
    return ok();
}

}  // extern "C"
