// Host-only driver for the GGUF reader under AddressSanitizer: opens every
// file named on the command line, looks up each tensor and touches its bytes.
// Built by tests/test_gguf.py with g++ -fsanitize=address together with
// q2k_gguf.cpp and a stand-in for the library's error-message functions.
#include <cstdarg>
#include <cstdio>

#include "q2k.h"
#include "q2k_error.h"

namespace q2k {
static char msg[512];
q2k_status set_error_v(q2k_status s, const char *fmt, va_list ap) {
    std::vsnprintf(msg, sizeof msg, fmt, ap);
    return s;
}
void clear_error() { msg[0] = '\0'; }
}  // namespace q2k

int main(int argc, char **argv) {
    unsigned long long opened = 0, touched = 0;
    for (int i = 1; i < argc; ++i) {
        q2k_gguf *f = nullptr;
        if (q2k_gguf_open(argv[i], &f) != Q2K_OK) continue;
        ++opened;
        for (uint64_t t = 0; t < q2k_gguf_tensor_count(f); ++t) {
            const char *name = q2k_gguf_tensor_name(f, t);
            q2k_gguf_info info;
            if (q2k_gguf_tensor_info(f, name, &info) != Q2K_OK) continue;
            const void *data;
            uint64_t n;
            if (q2k_gguf_tensor_data(f, name, &data, &n) != Q2K_OK) continue;
            const unsigned char *p = static_cast<const unsigned char *>(data);
            unsigned sum = 0;
            for (uint64_t k = 0; k < n; ++k) sum += p[k];
            touched += n + (sum & 0);
        }
        q2k_gguf_close(f);
    }
    std::printf("opened %llu touched %llu\n", opened, touched);
    return 0;
}
