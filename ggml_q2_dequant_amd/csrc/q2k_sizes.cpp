// Host-side sizes of the kernels' work splits and device scratch: how the
// argmax path cuts a row into chunks and how the expert-routed matrix-core
// schedule lays out its scratch buffer. Plain C++ with no device code, so the
// validation layer (q2k_api.cpp) also builds with a host compiler alone.
#include <stdint.h>

#include "q2k_launch.h"

namespace q2k {

namespace {

constexpr uint64_t align256(uint64_t v) { return (v + 255u) & ~uint64_t{255u}; }

}  // namespace

uint32_t sample_chunk(uint32_t vocab) {
    // 256 threads x at least 16 columns each, and at most kSampleMaxChunks
    // chunks per slot; a multiple of 256 so each wavefront's quarter is whole
    // 64-column steps.
    uint64_t chunk = (static_cast<uint64_t>(vocab) + kSampleMaxChunks - 1) / kSampleMaxChunks;
    if (chunk < 4096) chunk = 4096;
    chunk = (chunk + 255) / 256 * 256;
    return static_cast<uint32_t>(chunk);
}

uint64_t sample_workspace_bytes(uint32_t n_slots, uint32_t vocab) {
    // Per slot and chunk: one partial maximum, the kept local candidates and
    // their count.
    const uint32_t chunk = sample_chunk(vocab);
    const uint64_t chunks = (vocab + chunk - 1) / chunk;
    return static_cast<uint64_t>(n_slots) * chunks *
           (kSampleArgMaxBytes + kSampleLocalCap * kSampleCandBytes + sizeof(uint32_t));
}

uint32_t moe_tiles_max(uint32_t routes, uint32_t n_experts) {
    // sum over non-empty experts of ceil(count / 128) <= (routes + 127 * non-empty experts) / 128
    const uint64_t used = routes < n_experts ? routes : n_experts;
    return static_cast<uint32_t>((routes + used * (kMoeTileRows - 1)) / kMoeTileRows);
}

uint64_t moe_scratch_bytes(uint32_t routes, uint32_t n_experts, uint32_t K) {
    return align256(16) + align256(4ull * routes) + align256(sizeof(MoeTile) * moe_tiles_max(routes, n_experts)) +
           2ull * routes * K;
}

MoeScratch moe_scratch_carve(void *base, uint32_t routes, uint32_t n_experts) {
    auto *b = static_cast<uint8_t *>(base);
    MoeScratch s;
    s.hdr = reinterpret_cast<uint32_t *>(b);
    b += align256(16);
    s.perm = reinterpret_cast<uint32_t *>(b);
    b += align256(4ull * routes);
    s.tiles = reinterpret_cast<MoeTile *>(b);
    b += align256(sizeof(MoeTile) * moe_tiles_max(routes, n_experts));
    s.x_bf16 = b;
    return s;
}

}  // namespace q2k
