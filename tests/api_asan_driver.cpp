// Host-only driver for the C ABI layer (q2k_api.cpp) built with g++ under
// AddressSanitizer + UBSan, or ThreadSanitizer, against tests/asan_stubs.cpp
// (host memory instead of device memory, launch stubs that touch exactly the
// bytes each kernel touches).
//
// Every buffer is allocated at exactly the size include/q2k.h states for the
// call, so a call that lets a kernel reach past a buffer, or sizes a
// workspace or caller scratch too small for the layout its kernels use, is a
// heap-buffer-overflow here. Covered: every entry point's accepted path
// (workspace growth over a sequence of sizes, the pooled forms with
// exactly-sized scratch, the no-allocation form, argmax calls split over
// several launches, the expert-routed schedules with bad ids and padded
// expert strides, the gather's status word), growth refused during a graph
// capture, and calls from several host threads at once on shared and
// separate streams. Prints "ok <checks> <launches>" and exits 0, or lists
// each failed expectation and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "q2k.h"

extern "C" {
void stub_set_capturing(int on);
void stub_fail_gather_done(int on);
unsigned long long stub_launches(void);
unsigned long long stub_mallocs(void);
}

namespace {

int g_checks = 0, g_fail = 0;

#define EXPECT(cond, ...)                                                                   \
    do {                                                                                    \
        ++g_checks;                                                                         \
        if (!(cond)) {                                                                      \
            ++g_fail;                                                                       \
            std::fprintf(stderr, "FAIL line %d: ", __LINE__);                              \
            std::fprintf(stderr, __VA_ARGS__);                                              \
            std::fprintf(stderr, " [last error: %s]\n", q2k_last_error_message());         \
        }                                                                                   \
    } while (0)

// An exactly-sized, 256-byte aligned heap block.
struct Buf {
    void *p = nullptr;
    size_t n = 0;
    explicit Buf(size_t bytes) : n(bytes) {
        if (posix_memalign(&p, 256, bytes ? bytes : 1) != 0) std::abort();
        std::memset(p, 0, bytes);
    }
    ~Buf() { std::free(p); }
    Buf(const Buf &) = delete;
    Buf &operator=(const Buf &) = delete;
    template <class T>
    T *as() const {
        return static_cast<T *>(p);
    }
};

void *stream(uintptr_t i) { return reinterpret_cast<void *>(i * 0x1000); }

uint64_t wbytes(uint64_t rows, uint32_t K) { return rows * (K / 256) * 84; }

void matmul_case(uint32_t M, uint32_t N, uint32_t K, void *st) {
    Buf x(4ull * M * K), w(wbytes(N, K)), y(4ull * M * N);
    const q2k_path paths[3] = {Q2K_PATH_AUTO, Q2K_PATH_GEMV, Q2K_PATH_MFMA};
    for (q2k_path path : paths) {
        if (path == Q2K_PATH_GEMV && M > 8) continue;
        q2k_status s = q2k_matmul_path(x.as<float>(), w.p, y.as<float>(), M, N, K, path, st);
        EXPECT(s == Q2K_OK, "matmul M=%u N=%u K=%u path=%d: %d", M, N, K, path, s);
        uint64_t need = ~0ull;
        s = q2k_matmul_scratch_bytes(M, N, K, path, &need);
        EXPECT(s == Q2K_OK, "scratch_bytes M=%u K=%u", M, K);
        Buf scratch(need);
        s = q2k_matmul_pooled(x.as<float>(), w.p, y.as<float>(), M, N, K, path, need ? scratch.p : nullptr, need, st);
        EXPECT(s == Q2K_OK, "pooled M=%u N=%u K=%u path=%d: %d", M, N, K, path, s);
        if (need) {
            s = q2k_matmul_pooled(x.as<float>(), w.p, y.as<float>(), M, N, K, path, scratch.p, need - 1, st);
            EXPECT(s == Q2K_ERR_INVALID_ARGUMENT, "pooled with one byte short must be rejected");
        }
    }
    const q2k_status s = q2k_matmul_noalloc(x.as<float>(), w.p, y.as<float>(), M, N, K, st);
    EXPECT(s == Q2K_OK, "noalloc M=%u N=%u K=%u: %d", M, N, K, s);
}

void matmul_cases() {
    const uint32_t shapes[][3] = {{1, 33, 256}, {2, 64, 512}, {3, 17, 768}, {8, 5, 256},   {9, 40, 512},
                                  {40, 30, 768}, {300, 7, 256}, {17, 3, 1024}, {1, 1, 4096}, {129, 2, 512}};
    for (auto &sh : shapes) matmul_case(sh[0], sh[1], sh[2], stream(1));
    // Workspace growth on one stream: small, larger, much larger, smaller again.
    for (uint32_t M : {16u, 24u, 200u, 12u, 640u, 64u}) matmul_case(M, 8, 512, stream(2));

    // The no-allocation form refuses more bf16 activations than its array holds.
    const uint32_t K = 1024, M = (16u << 20) / (2 * K) + 1;
    Buf x(4ull * M * K), w(wbytes(4, K)), y(4ull * M * 4);
    EXPECT(q2k_matmul_noalloc(x.as<float>(), w.p, y.as<float>(), M, 4, K, stream(1)) == Q2K_ERR_INVALID_ARGUMENT &&
               std::strstr(q2k_last_error_message(), "device scratch holds"),
           "noalloc over its array must be rejected");
    EXPECT(q2k_matmul_noalloc(x.as<float>(), w.p, y.as<float>(), M - 1, 4, K, stream(1)) == Q2K_OK,
           "noalloc at its array's size");

    Buf xb(4ull * 3 * 2 * 512), wb(wbytes(3ull * 10, 512)), yb(4ull * 3 * 2 * 10);
    EXPECT(q2k_matmul_batched(xb.as<float>(), wb.p, yb.as<float>(), 3, 2, 10, 512, stream(1)) == Q2K_OK, "batched");
    Buf x1(4ull * 65537 * 256), w1(wbytes(65537ull, 256)), y1(4ull * 65537);
    EXPECT(q2k_matmul_batched(x1.as<float>(), w1.p, y1.as<float>(), 65537, 1, 1, 256, stream(1)) == Q2K_OK,
           "batched over two launches");
}

void dequant_and_gather_cases() {
    Buf blocks(3 * 84), out(4 * 768);
    EXPECT(q2k_dequantize(blocks.p, 3 * 84, out.as<float>(), 768, stream(1)) == Q2K_OK, "dequantize");

    const uint32_t vocab = 10, dim = 512, nt = 5;
    Buf table(wbytes(vocab, dim)), ids(4 * nt), emb(4ull * nt * dim), status(4);
    for (uint32_t t = 0; t < nt; ++t) ids.as<uint32_t>()[t] = (t * 7) % vocab;
    EXPECT(q2k_embedding_gather(table.p, ids.as<uint32_t>(), emb.as<float>(), vocab, dim, nt, stream(1)) == Q2K_OK,
           "gather");
    ids.as<uint32_t>()[3] = vocab;
    EXPECT(q2k_embedding_gather(table.p, ids.as<uint32_t>(), emb.as<float>(), vocab, dim, nt, stream(1)) ==
               Q2K_ERR_ID_OUT_OF_RANGE,
           "gather with an id >= vocab");
    ids.as<uint32_t>()[3] = 0;
    EXPECT(q2k_embedding_gather(table.p, ids.as<uint32_t>(), emb.as<float>(), vocab, dim, nt, stream(1)) == Q2K_OK,
           "gather after a failed call starts from a clear status word");
    // A failed completion launch after a gather that saw a bad id: the next call clears the status word
    // first and succeeds.
    ids.as<uint32_t>()[2] = vocab + 5;
    stub_fail_gather_done(1);
    EXPECT(q2k_embedding_gather(table.p, ids.as<uint32_t>(), emb.as<float>(), vocab, dim, nt, stream(1)) ==
               Q2K_ERR_DEVICE,
           "gather whose completion launch fails");
    stub_fail_gather_done(0);
    ids.as<uint32_t>()[2] = 1;
    EXPECT(q2k_embedding_gather(table.p, ids.as<uint32_t>(), emb.as<float>(), vocab, dim, nt, stream(1)) == Q2K_OK,
           "gather after a failed completion launch");
    ids.as<uint32_t>()[0] = 0xFFFFFFFFu;
    EXPECT(q2k_embedding_gather_async(table.p, ids.as<uint32_t>(), emb.as<float>(), vocab, dim, nt,
                                      status.as<int>(), stream(1)) == Q2K_OK &&
               *status.as<int>() == 1,
           "gather_async reports a bad id in the status word");
}

void argmax_case(uint32_t ns, uint32_t vocab, uint32_t cap, void *st) {
    Buf lg(4ull * ns * vocab), i1(4ull * ns), v1(4ull * ns), cnt(4ull * ns), ovf(4ull * ns), ids(4ull * ns * cap);
    q2k_status s = q2k_argmax_candidates(lg.as<float>(), ns, vocab, cap, i1.as<uint32_t>(), v1.as<float>(),
                                         cnt.as<uint32_t>(), ovf.as<uint32_t>(), ids.as<uint32_t>(), st);
    EXPECT(s == Q2K_OK, "argmax ns=%u vocab=%u", ns, vocab);
    uint64_t need = 0;
    EXPECT(q2k_argmax_candidates_scratch_bytes(ns, vocab, &need) == Q2K_OK && need > 0, "argmax scratch bytes");
    Buf scratch(need);
    s = q2k_argmax_candidates_pooled(lg.as<float>(), ns, vocab, cap, i1.as<uint32_t>(), v1.as<float>(),
                                     cnt.as<uint32_t>(), ovf.as<uint32_t>(), ids.as<uint32_t>(), scratch.p, need, st);
    EXPECT(s == Q2K_OK, "argmax pooled ns=%u vocab=%u", ns, vocab);
}

void argmax_cases() {
    argmax_case(3, 70001, 16, stream(3));
    argmax_case(1, 1, 1, stream(3));
    argmax_case(2, 262144, 4, stream(3));
    argmax_case(65537, 3, 2, stream(3));   // two launches share the scratch of the larger one
    argmax_case(1, 8193, 1, stream(3));
}

void moe_case(uint32_t n_tokens, uint32_t top_k, uint32_t n, uint32_t k, uint32_t n_experts, uint32_t pad,
              uint32_t n_bad, void *st) {
    q2k_matmul_id_params p{};
    p.n_tokens = n_tokens;
    p.top_k = top_k;
    p.n = n;
    p.k = k;
    p.n_experts = n_experts;
    p.expert_stride = wbytes(n, k) + pad;
    const uint64_t routes = static_cast<uint64_t>(n_tokens) * top_k;
    const uint64_t wb = (n_experts - 1) * p.expert_stride + wbytes(n, k);
    Buf x(4ull * n_tokens * k), xs(4ull * routes * k), w0(wb), w1(wb), ids(4 * routes), y0(4 * routes * n),
        y1(4 * routes * n), status(4);
    for (uint64_t r = 0; r < routes; ++r) ids.as<uint32_t>()[r] = static_cast<uint32_t>((r * 5 + r / 3) % n_experts);
    for (uint32_t b = 0; b < n_bad && b < routes; ++b) ids.as<uint32_t>()[(b * 13) % routes] = n_experts + b;
    const q2k_path paths[3] = {Q2K_PATH_AUTO, Q2K_PATH_GEMV, Q2K_PATH_MFMA};
    for (q2k_path path : paths) {
        *status.as<int>() = 0;
        const q2k_status s = q2k_matmul_id_path(x.as<float>(), w0.p, ids.as<uint32_t>(), y0.as<float>(), &p,
                                                status.as<int>(), path, st);
        EXPECT(s == Q2K_OK, "matmul_id tokens=%u top_k=%u path=%d: %d", n_tokens, top_k, path, s);
        EXPECT(*status.as<int>() == (n_bad ? 1 : 0), "matmul_id status word, path=%d", path);
    }
    const uint64_t need = q2k_matmul_id_scratch_bytes(&p);
    EXPECT(need > 0, "matmul_id scratch bytes");
    Buf scratch(need);
    EXPECT(q2k_matmul_id_pooled(x.as<float>(), w0.p, ids.as<uint32_t>(), y0.as<float>(), &p, scratch.p, need,
                                status.as<int>(), st) == Q2K_OK,
           "matmul_id pooled");
    EXPECT(q2k_matmul_id_pooled_pair(x.as<float>(), w0.p, w1.p, ids.as<uint32_t>(), y0.as<float>(), y1.as<float>(),
                                     &p, scratch.p, need, nullptr, st) == Q2K_OK,
           "matmul_id pooled pair");
    EXPECT(q2k_matmul_id_pooled_slotted(xs.as<float>(), w0.p, ids.as<uint32_t>(), y0.as<float>(), &p, scratch.p,
                                        need, status.as<int>(), st) == Q2K_OK,
           "matmul_id pooled slotted");
    EXPECT(q2k_matmul_id_pooled(x.as<float>(), w0.p, ids.as<uint32_t>(), y0.as<float>(), &p, scratch.p, need - 1,
                                status.as<int>(), st) == Q2K_ERR_INVALID_ARGUMENT,
           "matmul_id pooled one byte short must be rejected");
}

void moe_cases() {
    moe_case(3, 2, 16, 512, 4, 0, 0, stream(4));
    moe_case(40, 6, 24, 256, 8, 4, 3, stream(4));
    moe_case(300, 8, 8, 256, 64, 256, 0, stream(4));
    moe_case(130, 1, 4, 512, 1, 0, 1, stream(4));
    moe_case(33, 8, 4, 256, 512, 0, 5, stream(5));
}

void capture_cases() {
    Buf x(4ull * 64 * 512), w(wbytes(8, 512)), y(4ull * 64 * 8);
    // A stream whose workspace already holds 64 x 512 bf16 values.
    EXPECT(q2k_matmul(x.as<float>(), w.p, y.as<float>(), 64, 8, 512, stream(6)) == Q2K_OK, "eager call before capture");
    const unsigned long long before = stub_mallocs(), launches = stub_launches();
    stub_set_capturing(1);
    EXPECT(q2k_matmul(x.as<float>(), w.p, y.as<float>(), 64, 8, 512, stream(6)) == Q2K_OK,
           "captured call within the workspace");
    EXPECT(q2k_matmul(x.as<float>(), w.p, y.as<float>(), 32, 8, 512, stream(7)) == Q2K_ERR_INVALID_ARGUMENT &&
               std::strstr(q2k_last_error_message(), "graph capture"),
           "growth during capture must be refused");
    EXPECT(q2k_matmul(x.as<float>(), w.p, y.as<float>(), 1, 8, 512, stream(7)) == Q2K_OK,
           "a GEMV call needs no workspace during capture");
    Buf table(wbytes(4, 256)), ids(4 * 2), emb(4ull * 2 * 256);
    EXPECT(q2k_embedding_gather(table.p, ids.as<uint32_t>(), emb.as<float>(), 4, 256, 2, stream(7)) ==
               Q2K_ERR_INVALID_ARGUMENT,
           "the synchronous gather must be refused during capture");
    stub_set_capturing(0);
    EXPECT(stub_mallocs() == before, "no allocation during capture");
    EXPECT(stub_launches() == launches + 2, "the refused call enqueued nothing");
}

void thread_cases() {
    // Four threads on one stream (the workspace lock serialises growth and the
    // launches that use it) and four on streams of their own.
    std::vector<std::thread> th;
    for (int t = 0; t < 8; ++t) {
        th.emplace_back([t] {
            void *st = stream(t < 4 ? 100 : 101 + t);
            for (int i = 0; i < 6; ++i) {
                const uint32_t M = 9 + 37 * ((t + i) % 5);
                Buf x(4ull * M * 256), w(wbytes(3, 256)), y(4ull * M * 3);
                if (q2k_matmul(x.as<float>(), w.p, y.as<float>(), M, 3, 256, st) != Q2K_OK) std::abort();
                Buf lg(4ull * 2 * 9000), o(4ull * (4 * 2 + 2 * 3));
                auto *u = o.as<uint32_t>();
                if (q2k_argmax_candidates(lg.as<float>(), 2, 9000, 3, u, o.as<float>() + 2, u + 4, u + 6, u + 8, st) !=
                    Q2K_OK)
                    std::abort();
            }
        });
    }
    for (auto &t : th) t.join();
    ++g_checks;
}

}  // namespace

int main(int argc, char **argv) {
    const bool threads_only = argc > 1 && std::strcmp(argv[1], "--threads") == 0;
    if (!threads_only) {
        matmul_cases();
        dequant_and_gather_cases();
        argmax_cases();
        moe_cases();
        capture_cases();
    }
    thread_cases();
    if (g_fail) {
        std::fprintf(stderr, "%d of %d checks failed\n", g_fail, g_checks);
        return 1;
    }
    std::printf("ok %d %llu\n", g_checks, stub_launches());
    return 0;
}
