// Internal launch interface between the C ABI (q2k_api.cpp) and the HIP
// kernels (q2k_kernels.hip). Arguments are validated by the caller; these
// functions only size grids and enqueue kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q2k_error.h"

namespace q2k {

constexpr uint32_t kQK = 256;          // weights per super-block
constexpr uint32_t kBlockBytes = 84;   // bytes per super-block
constexpr uint32_t kGemvMaxM = 8;      // largest M the fp32 GEMV handles
constexpr uint32_t kMaxK = 1u << 21;   // keeps every per-workgroup byte offset below 2^31
constexpr uint32_t kMaxGridY = 65535;  // largest batch count one GEMV launch takes

hipError_t launch_dequantize(const uint8_t *blocks, uint64_t nblocks, float *out, hipStream_t stream);

// A bad id (>= vocab) makes the kernel store bad_value into *status.
hipError_t launch_gather(const uint8_t *table, const uint32_t *ids, float *out, uint32_t vocab,
                         uint32_t blocks_per_row, uint32_t n_tokens, int *status, int bad_value, hipStream_t stream);

// Queued after launch_gather on the same stream, so it starts once the gather
// kernel has ended: one thread clears *status and then stores
// (seq << 2) | 2 | (*status was seq) into *host_word (host-visible memory,
// system scope, release), which the host can poll for the end of the gather
// and its id check.
hipError_t launch_gather_done(int *status, int seq, int *host_word, hipStream_t stream);

// 1 <= M <= 8; batches problems laid out batch-major (x [batches, M, K],
// w [batches, N, K/256 blocks], y [batches, M, N]), 1 <= batches <= kMaxGridY.
// Needs no workspace.
hipError_t launch_gemv(const float *x, const uint8_t *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                       uint32_t batches, hipStream_t stream);

// Matrix-core path. x_bf16 is a device workspace of at least M * K * 2 bytes
// (16-byte aligned) that receives bf16(x) before the GEMM reads it.
hipError_t launch_gemm_mfma(const float *x, const uint8_t *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                            void *x_bf16, hipStream_t stream);

// q2k_matmul_noalloc (q2k_noalloc.hip): the device address of the library's
// file-scope scratch array on the current device, kNoAllocScratchBytes long,
// 256-byte aligned; looked up once per device, never allocated.
constexpr uint64_t kNoAllocScratchBytes = 16ull << 20;
hipError_t noalloc_scratch(void **out);

// First-max argmax + threshold candidates over [n_slots, vocab] logits
// (q2k_sample.hip). workspace holds sample_workspace_bytes(n_slots, vocab)
// bytes, 8-byte aligned; 1 <= n_slots <= kMaxGridY, vocab, cap >= 1. Its
// layout, per (slot, chunk) in slot-major order: all the chunk partials
// (value, index), then all the kept local candidates (kSampleLocalCap of
// (index, value) each), then all the local candidate counts (u32).
// sample_chunk and the scratch sizes below are host code (q2k_sizes.cpp).
constexpr uint32_t kSampleMaxChunks = 64;      // chunks (workgroups) per slot
constexpr uint32_t kSampleMaxVocab = 1u << 29;  // keeps every row's byte offsets below 2^31
constexpr uint32_t kSampleArgMaxBytes = 8;     // one chunk's partial: value and index
constexpr uint32_t kSampleLocalCap = 64;       // local candidates kept per chunk
constexpr uint32_t kSampleCandBytes = 8;       // one kept candidate: index and value
uint32_t sample_chunk(uint32_t vocab);
uint64_t sample_workspace_bytes(uint32_t n_slots, uint32_t vocab);
hipError_t launch_argmax_candidates(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                    uint32_t *top1_idx, float *top1_val, uint32_t *cand_count, uint32_t *overflow,
                                    uint32_t *cand_ids, void *workspace, hipStream_t stream);

// Expert-routed product (routing and row gather in q2k_moe.hip, the routed
// modes of the GEMV and GEMM kernels in q2k_kernels.hip). Route r of
// n_tokens * top_k takes expert ids[r] and activation row r / x_div (x_div =
// top_k, or 1 when every route has its own row); its output row is r.
constexpr uint32_t kMoeMaxExperts = 512;     // LDS tables of the routing kernel
constexpr uint32_t kMoeMaxRoutes = 1u << 24;
constexpr uint32_t kMoeTileRows = 128;       // rows of one matrix-core tile

struct MoeTile {
    uint32_t expert, p0, count;  // rows p0 .. p0 + count - 1 of the expert-ordered list; count 0 = unused
};

// Device arrays carved from one scratch buffer (moe_scratch_bytes long).
struct MoeScratch {
    uint32_t *hdr;    // [4]: valid routes, tiles in use, routes with a bad id
    uint32_t *perm;   // [routes]: the route at each row of the expert order, then the bad routes
    MoeTile *tiles;   // [moe_tiles_max]
    void *x_bf16;     // [routes, K] bf16 activations in expert order
};
uint32_t moe_tiles_max(uint32_t routes, uint32_t n_experts);
uint64_t moe_scratch_bytes(uint32_t routes, uint32_t n_experts, uint32_t K);
MoeScratch moe_scratch_carve(void *base, uint32_t routes, uint32_t n_experts);

// fp32 path: one M = 1 GEMV per route; a route with a bad id gets a NaN row.
hipError_t launch_moe_gemv(const float *x, const uint8_t *w, const uint32_t *ids, float *y, uint32_t routes,
                           uint32_t x_div, uint32_t N, uint32_t K, uint32_t n_experts, uint64_t expert_stride,
                           int *status, hipStream_t stream);
// Matrix-core path, step 1: group routes by expert (stable), build the tile list.
hipError_t launch_moe_route(const uint32_t *ids, uint32_t routes, uint32_t n_experts, MoeScratch s, int *status,
                            hipStream_t stream);
// Step 2: bf16 activations in expert order; NaN rows of y0 (and y1) for bad ids.
hipError_t launch_moe_gather(const float *x, uint32_t routes, uint32_t x_div, uint32_t K, MoeScratch s, float *y0,
                             float *y1, uint32_t N, hipStream_t stream);
// Step 3: the tiles' products, written to their routes' rows of y.
hipError_t launch_moe_gemm(const uint8_t *w, float *y, uint32_t routes, uint32_t N, uint32_t K, uint32_t n_experts,
                           uint64_t expert_stride, MoeScratch s, hipStream_t stream);

}  // namespace q2k
