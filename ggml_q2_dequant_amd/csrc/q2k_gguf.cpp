// GGUF tensor directory reader: the host side that lets Q2_K weights stored
// in a GGUF file reach the kernels.
//
// Format facts used (from the file layout the docs.rs source page of
// mlx-native 0.10.8, tests/deepseek_q2_k.rs, writes in test
// q2_k_gguf_type_10_parses_with_exact_block_size, and the GGUF layout it
// follows):
//   "GGUF" magic, u32 version (2 and 3 use 64-bit counts), u64 tensor count,
//   u64 metadata key/value count; each key/value is a string key, a u32
//   value type and the value; each tensor record is a string name, u32
//   n_dims, n_dims u64 extents (fastest first), u32 type, u64 offset into the
//   data section; the data section starts at the next multiple of the
//   alignment (32, or the u32 metadata value "general.alignment").
//   Strings are a u64 byte length followed by the bytes. All integers are
//   little endian. Type 10 is Q2_K: 256 weights per 84-byte super-block.
//
// The file is memory-mapped read-only; tensor data are handed out as
// pointers into the mapping, so a model's weights can be uploaded without an
// extra host copy. Every read is bounds-checked against the file size.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "q2k.h"
#include "q2k_error.h"

namespace {

q2k_status gguf_fail(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    q2k::set_error_v(Q2K_ERR_INVALID_ARGUMENT, fmt, ap);
    va_end(ap);
    return Q2K_ERR_INVALID_ARGUMENT;
}

struct Tensor {
    std::string name;
    uint32_t type = 0;
    uint32_t n_dims = 0;
    uint64_t dims[Q2K_GGUF_MAX_DIMS] = {1, 1, 1, 1};
    uint64_t offset = 0;  // from the start of the data section
};

// Bytes per element group for the types whose size this reader knows.
bool type_size(uint32_t type, uint64_t *group, uint64_t *group_bytes) {
    switch (type) {
        case 0: *group = 1; *group_bytes = 4; return true;     // F32
        case 1: *group = 1; *group_bytes = 2; return true;     // F16
        case 10: *group = 256; *group_bytes = 84; return true; // Q2_K
        case 30: *group = 1; *group_bytes = 2; return true;    // BF16
        default: return false;
    }
}

// Little-endian cursor over the mapping.
struct Cursor {
    const uint8_t *base;
    uint64_t size, pos = 0;
    bool ok = true;

    bool take(uint64_t n, const uint8_t **p) {
        if (!ok || n > size - pos) {
            ok = false;
            return false;
        }
        *p = base + pos;
        pos += n;
        return true;
    }
    uint64_t uint(unsigned bytes) {
        const uint8_t *p;
        if (!take(bytes, &p)) return 0;
        uint64_t v = 0;
        for (unsigned i = 0; i < bytes; ++i) v |= static_cast<uint64_t>(p[i]) << (8 * i);
        return v;
    }
    std::string str() {
        const uint64_t n = uint(8);
        const uint8_t *p;
        if (!take(n, &p)) return std::string();
        return std::string(reinterpret_cast<const char *>(p), n);
    }
};

// Byte width of a scalar metadata value type, 0 for string and array.
unsigned scalar_width(uint32_t t) {
    switch (t) {
        case 0: case 1: case 7: return 1;  // u8, i8, bool
        case 2: case 3: return 2;          // u16, i16
        case 4: case 5: case 6: return 4;  // u32, i32, f32
        case 10: case 11: case 12: return 8;  // u64, i64, f64
        default: return 0;
    }
}

// Skip one metadata value of type t; arrays nest at most `depth` deep.
bool skip_value(Cursor &c, uint32_t t, int depth) {
    if (const unsigned w = scalar_width(t)) {
        const uint8_t *p;
        return c.take(w, &p);
    }
    if (t == 8) {
        c.str();
        return c.ok;
    }
    if (t == 9 && depth > 0) {
        const uint32_t et = static_cast<uint32_t>(c.uint(4));
        const uint64_t n = c.uint(8);
        if (!c.ok) return false;
        if (const unsigned w = scalar_width(et)) {
            const uint8_t *p;
            if (n > (c.size - c.pos) / w) return c.ok = false;
            return c.take(n * w, &p);
        }
        for (uint64_t i = 0; i < n; ++i)
            if (!skip_value(c, et, depth - 1)) return false;
        return c.ok;
    }
    return c.ok = false;
}

}  // namespace

struct q2k_gguf {
    void *map = nullptr;
    uint64_t size = 0;
    uint32_t version = 0;
    uint64_t alignment = 32;
    uint64_t data_start = 0;
    std::vector<Tensor> tensors;
    std::unordered_map<std::string, size_t> by_name;
};

extern "C" {

q2k_status q2k_gguf_open(const char *path, q2k_gguf **out) {
    if (!path || !out) return gguf_fail("q2k_gguf_open: null pointer");
    *out = nullptr;
    const int fd = ::open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return gguf_fail("q2k_gguf_open: cannot open %s", path);
    struct stat st;
    if (fstat(fd, &st) != 0 || st.st_size < 24) {
        ::close(fd);
        return gguf_fail("q2k_gguf_open: %s is too short for a GGUF header", path);
    }
    void *map = mmap(nullptr, static_cast<size_t>(st.st_size), PROT_READ, MAP_PRIVATE, fd, 0);
    ::close(fd);
    if (map == MAP_FAILED) return gguf_fail("q2k_gguf_open: cannot map %s", path);

    auto *f = new q2k_gguf;
    f->map = map;
    f->size = static_cast<uint64_t>(st.st_size);
    auto bail = [&](q2k_status s) {
        munmap(f->map, f->size);
        delete f;
        return s;
    };
    Cursor c{static_cast<const uint8_t *>(map), f->size};
    const uint8_t *magic;
    c.take(4, &magic);
    if (std::memcmp(magic, "GGUF", 4) != 0) return bail(gguf_fail("q2k_gguf_open: bad magic (not a GGUF file)"));
    f->version = static_cast<uint32_t>(c.uint(4));
    if (f->version != 2 && f->version != 3)
        return bail(gguf_fail("q2k_gguf_open: GGUF version %u is not supported (2 or 3)", f->version));
    const uint64_t n_tensors = c.uint(8), n_kv = c.uint(8);
    // Every record takes at least 8 bytes; reject counts the file cannot hold.
    if (!c.ok || n_tensors > f->size / 8 || n_kv > f->size / 8)
        return bail(gguf_fail("q2k_gguf_open: implausible tensor or key/value count"));

    for (uint64_t i = 0; i < n_kv; ++i) {
        const std::string key = c.str();
        const uint32_t t = static_cast<uint32_t>(c.uint(4));
        if (!c.ok) break;
        if (key == "general.alignment" && t == 4) {
            f->alignment = c.uint(4);
            if (f->alignment == 0 || (f->alignment & (f->alignment - 1)) != 0)
                return bail(gguf_fail("q2k_gguf_open: general.alignment %llu is not a power of two",
                                      static_cast<unsigned long long>(f->alignment)));
        } else if (!skip_value(c, t, 4)) {
            return bail(gguf_fail("q2k_gguf_open: bad metadata value (type %u) for key '%s'", t, key.c_str()));
        }
    }
    if (!c.ok) return bail(gguf_fail("q2k_gguf_open: file ends inside the metadata"));

    f->tensors.reserve(static_cast<size_t>(n_tensors));
    for (uint64_t i = 0; i < n_tensors; ++i) {
        Tensor t;
        t.name = c.str();
        t.n_dims = static_cast<uint32_t>(c.uint(4));
        if (!c.ok) break;
        if (t.n_dims == 0 || t.n_dims > Q2K_GGUF_MAX_DIMS)
            return bail(gguf_fail("q2k_gguf_open: tensor '%s' has %u dimensions (1..%d supported)", t.name.c_str(),
                                  t.n_dims, Q2K_GGUF_MAX_DIMS));
        for (uint32_t d = 0; d < t.n_dims; ++d) t.dims[d] = c.uint(8);
        t.type = static_cast<uint32_t>(c.uint(4));
        t.offset = c.uint(8);
        if (!c.ok) break;
        if (f->by_name.count(t.name)) return bail(gguf_fail("q2k_gguf_open: duplicate tensor '%s'", t.name.c_str()));
        f->by_name.emplace(t.name, f->tensors.size());
        f->tensors.push_back(std::move(t));
    }
    if (!c.ok) return bail(gguf_fail("q2k_gguf_open: file ends inside the tensor records"));
    f->data_start = (c.pos + f->alignment - 1) / f->alignment * f->alignment;
    *out = f;
    q2k::clear_error();
    return Q2K_OK;
}

void q2k_gguf_close(q2k_gguf *f) {
    if (!f) return;
    munmap(f->map, f->size);
    delete f;
}

uint64_t q2k_gguf_tensor_count(const q2k_gguf *f) { return f ? f->tensors.size() : 0; }

const char *q2k_gguf_tensor_name(const q2k_gguf *f, uint64_t index) {
    if (!f || index >= f->tensors.size()) return nullptr;
    return f->tensors[index].name.c_str();
}

q2k_status q2k_gguf_tensor_info(const q2k_gguf *f, const char *name, q2k_gguf_info *info) {
    if (!f || !name || !info) return gguf_fail("q2k_gguf_tensor_info: null pointer");
    const auto it = f->by_name.find(name);
    if (it == f->by_name.end()) return gguf_fail("q2k_gguf_tensor_info: no tensor named '%s'", name);
    const Tensor &t = f->tensors[it->second];
    std::memset(info, 0, sizeof *info);
    info->ggml_type = t.type;
    info->n_dims = t.n_dims;
    uint64_t elems = 1;
    bool overflow = false;
    for (uint32_t d = 0; d < Q2K_GGUF_MAX_DIMS; ++d) {
        info->dims[d] = t.dims[d];
        if (d < t.n_dims) {
            if (t.dims[d] != 0 && elems > UINT64_MAX / t.dims[d]) overflow = true;
            elems *= t.dims[d];
        }
    }
    info->file_offset = f->data_start + t.offset;
    uint64_t group, gbytes;
    if (overflow || !type_size(t.type, &group, &gbytes)) {
        info->byte_len = 0;  // size unknown to this reader
    } else {
        if (t.dims[0] % group != 0)
            return gguf_fail("q2k_gguf_tensor_info: '%s' has %llu elements per row, not a multiple of %llu",
                             name, static_cast<unsigned long long>(t.dims[0]), static_cast<unsigned long long>(group));
        info->byte_len = elems / group * gbytes;
    }
    if (info->file_offset > f->size || info->byte_len > f->size - info->file_offset)
        return gguf_fail("q2k_gguf_tensor_info: '%s' lies outside the file", name);
    q2k::clear_error();
    return Q2K_OK;
}

q2k_status q2k_gguf_tensor_data(const q2k_gguf *f, const char *name, const void **data, uint64_t *byte_len) {
    if (!data || !byte_len) return gguf_fail("q2k_gguf_tensor_data: null pointer");
    q2k_gguf_info info;
    q2k_status s = q2k_gguf_tensor_info(f, name, &info);
    if (s != Q2K_OK) return s;
    if (info.byte_len == 0) return gguf_fail("q2k_gguf_tensor_data: the size of type %u is unknown", info.ggml_type);
    *data = static_cast<const uint8_t *>(f->map) + info.file_offset;
    *byte_len = info.byte_len;
    return Q2K_OK;
}

}  // extern "C"
