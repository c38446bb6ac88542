/*
 * q2k.h — C ABI of libq2k, the MI355X (gfx950) Q2_K weight path.
 *
 * Q2_K is GGML's 2-bit k-quant. Its layout and decode rule are those of the
 * docs.rs source page of mlx-native 0.10.8, tests/deepseek_q2_k.rs
 * (constants QK_K and BLOCK_BYTES, fn block, fn reference_dequant):
 *
 *   one super-block = 256 weights in 84 bytes
 *     bytes  0..15  scales[16]  low nibble: sub-block scale sc, high nibble: sub-block min mn
 *     bytes 16..79  qs[64]      2-bit codes, four per byte
 *     bytes 80..81  d           IEEE f16, little endian
 *     bytes 82..83  dmin        IEEE f16, little endian
 *   weight e (0..255): s = scales[e / 16], q = (qs[32*(e/128) + e%32] >> 2*((e/32)%4)) & 3,
 *                      w = f32(d)*sc*q - f32(dmin)*mn, evaluated in f32.
 *
 * A weight matrix W[N, K] (K a multiple of 256) is N rows of K/256 blocks, row
 * after row, blocks of a row in increasing k (fn run_dense appends the blocks
 * of each row in turn). An embedding table [vocab, embed_dim] is the same with
 * vocab rows.
 *
 * Conventions shared by every call:
 *  - Every pointer is caller-owned DEVICE memory on the current HIP device.
 *    libq2k never frees or retains it.
 *  - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on it;
 *    q2k_dequantize and q2k_matmul return before the GPU finishes, so the caller
 *    synchronises before reading outputs (the page's encode / commit_and_wait
 *    split). q2k_embedding_gather waits for its own kernel (see below).
 *  - All arguments are validated before anything is enqueued. On any error the
 *    call returns a non-zero status, enqueues nothing and leaves outputs
 *    untouched (except the gather's out-of-range case, documented below);
 *    q2k_last_error_message() then describes the failure.
 *  - Alignment: float outputs and x must be 16-byte aligned; Q2_K byte buffers
 *    and ids must be 4-byte aligned (84 is a multiple of 4).
 *  - An output range may not overlap any input range.
 *  - Calls on different streams may run concurrently; each call only reads its
 *    inputs and writes its outputs.
 *  - Device scratch. Three kinds of call stage data in device scratch: the
 *    matrix-core matmul (bf16(x)), the matrix-core expert-routed schedule and
 *    the argmax/candidate call. Each has a *_pooled form that takes
 *    caller-owned scratch and allocates nothing. The plain forms use a
 *    workspace libq2k keeps per (device, stream): hipMalloc'd when a call needs
 *    more than it holds (growing to at least twice its size); a call holds it
 *    from its size check until its kernels are enqueued; a buffer that growth
 *    replaces is retired but never freed before the process ends, so a graph
 *    captured earlier keeps a valid address. Growth is refused with
 *    Q2K_ERR_INVALID_ARGUMENT while the stream is capturing a graph: capture
 *    after one call of the largest size, or use the pooled form. A replayed
 *    graph shares the workspace with later calls on its capture stream, so the
 *    two must not run at the same time.
 */
#ifndef Q2K_H
#define Q2K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q2K_QK 256          /* weights per super-block */
#define Q2K_BLOCK_BYTES 84  /* bytes per super-block */

typedef enum q2k_status {
    Q2K_OK = 0,
    Q2K_ERR_INVALID_ARGUMENT = 1, /* bad size, null or misaligned pointer, overlap */
    Q2K_ERR_ID_OUT_OF_RANGE = 2,  /* q2k_embedding_gather: some id >= vocab */
    Q2K_ERR_DEVICE = 3            /* a HIP runtime call failed */
} q2k_status;

/* Matmul kernel choice. Q2K_PATH_AUTO picks the fp32 GEMV for M <= 8 and the
 * bf16 matrix-core path for M > 8, the switch the page's dense test makes at
 * more than 8 rows (fn run_dense: its tolerance changes there). The forced
 * values mirror the page's forced-mm test hooks (dispatch_mm_for_test).
 * Passed as an int: any other value is rejected with Q2K_ERR_INVALID_ARGUMENT
 * (in C++ the type is given int as its underlying type, so such a value is
 * still a valid q2k_path to receive and test). */
#ifdef __cplusplus
typedef enum q2k_path : int {
#else
typedef enum q2k_path {
#endif
    Q2K_PATH_AUTO = 0,
    Q2K_PATH_GEMV = 1, /* fp32 GEMV; only valid for 1 <= M <= 8 */
    Q2K_PATH_MFMA = 2  /* bf16 operands (round to nearest even), fp32 accumulation; any M */
} q2k_path;

/*
 * q2k_dequantize — decode whole Q2_K blocks to f32.
 * Page: test q2_k_host_decode_matches_all_256_canonical_values (values) and
 * test q2_k_host_decode_rejects_malformed_buffers (length rules).
 *   blocks       device bytes, blocks_bytes long; 4-byte aligned.
 *   blocks_bytes must be a positive multiple of 84.
 *   out          device f32 [out_elems]; 16-byte aligned.
 *   out_elems    must equal blocks_bytes / 84 * 256.
 * out[256*b + e] = weight e of block b, bit-identical to the f32 decode rule
 * above (the value is unique: d*sc*q and dmin*mn are exact in f32, only the
 * final subtraction rounds). Asynchronous on `stream`.
 */
q2k_status q2k_dequantize(const void *blocks, size_t blocks_bytes, float *out, size_t out_elems,
                          void *stream);

/*
 * q2k_matmul — y[M, N] = x[M, K] * W[N, K]^T with W in Q2_K.
 * Page: fn run_dense, which calls quantized_matmul_ggml with (m, n, k).
 *   x  device f32 [M, K] row-major; 16-byte aligned.
 *   w  device Q2_K bytes, N * K/256 * 84 long (layout above); 4-byte aligned.
 *   y  device f32 [M, N] row-major; 16-byte aligned.
 *   M, N >= 1; K a multiple of 256 with 256 <= K <= 2^21.
 * M <= 8 runs an fp32 GEMV (no workspace). Both forms compute each block as
 * d * sum(x * sc*q) - dmin * sum_s(mn_s * sum_{k in s} x), so their error is
 * stated against B = sum_k |x[k]| * (|d*sc*q| + |dmin*mn|), which equals
 * A = sum_k |x*w| unless a block's code and min terms cancel:
 *  - M <= 2 (fp32 FMAs on exact encodings of the codes):
 *      |y - exact| <= (27 + 2*ceil(K/4096)) * 2^-24 * B  (first order),
 *    for activations above about 2^-100 wherever they meet a non-zero code.
 *    This is within 1e-5 * A whenever B <= 5.5 * A (K <= 4096). A block whose
 *    weights are all exactly zero still contributes up to that bound times its B.
 *  - 3 <= M <= 8 (matrix cores on exact f16 encodings of sc*q and of mn, x
 *    scaled per block row and split into two f16 pieces): the matrix cores
 *    sum the 32 products of each step within a window of about 2^16 below
 *    its largest product, and the split keeps about 22 bits of each
 *    activation above 2^-34 of its block row's largest. So
 *      |y - exact| <= 2^-18 * B + 2^-6 * sum_b max_{k in b}|x[k]| *
 *                     (max_{k in b} |d*sc*q| + 16 * max_{s in b} |dmin*mn_s|),
 *    which is within 1e-5 * A as for M <= 2 whenever the activations of each
 *    256-weight block span less than 2^10 in magnitude (every product then
 *    lies inside the window); beyond that small activations lose precision
 *    relative to their block's largest.
 * A row of y depends only on its own row of x: calls with the same M give it
 * bit-identical values whatever the other rows hold (M <= 2 and 3 <= M <= 8
 * run different kernels and may differ in the last bits).
 * M > 8 runs the matrix-core path on bf16(x) and bf16(w) with fp32
 * accumulation: |y - exact| <= 4e-3 * sum_k |x*w| + 1e-6. That path stages
 * bf16(x) (2 * M * K bytes) in the stream's workspace (conventions above);
 * q2k_matmul_pooled takes it from the caller instead.
 * Asynchronous on `stream`.
 */
q2k_status q2k_matmul(const float *x, const void *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                      void *stream);

/* q2k_matmul with an explicit kernel choice (see q2k_path). Same arguments,
 * rules and guarantees; Q2K_PATH_GEMV with M > 8 is Q2K_ERR_INVALID_ARGUMENT. */
q2k_status q2k_matmul_path(const float *x, const void *w, float *y, uint32_t M, uint32_t N,
                           uint32_t K, q2k_path path, void *stream);

/* q2k_matmul_scratch_bytes — device scratch q2k_matmul_pooled needs for these
 * sizes and path: 2 * M * K bytes (bf16(x)) for the matrix-core path, 0 for
 * the GEMV. Shape rules as for q2k_matmul (pointers aside); *bytes is written
 * only on success. */
q2k_status q2k_matmul_scratch_bytes(uint32_t M, uint32_t N, uint32_t K, q2k_path path, uint64_t *bytes);

/* q2k_matmul_pooled — q2k_matmul_path with caller-held scratch and no
 * allocation (page: the pooled calls' caller-provided IdMmScratch, applied to
 * the dense product). When the path needs scratch, `scratch` is device memory
 * of at least q2k_matmul_scratch_bytes bytes, 256-byte aligned, not
 * overlapping x, w or y; its contents on entry do not matter and it is in use
 * until the call's work on `stream` ends. When the path needs none (the GEMV),
 * scratch and scratch_bytes are ignored. Same results, bit for bit, as
 * q2k_matmul_path with the same path. */
q2k_status q2k_matmul_pooled(const float *x, const void *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                             q2k_path path, void *scratch, uint64_t scratch_bytes, void *stream);

/*
 * q2k_matmul_noalloc — q2k_matmul for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, kernel choice, rules and results, bit for
 * bit, as q2k_matmul. It calls no allocating routine: for M > 8 it stages
 * bf16(x) in a device array compiled into libq2k (16 MiB per GPU, held until
 * the process ends), so M > 8 requires 2 * M * K <= 16 MiB (M * K <= 8388608);
 * larger sizes are Q2K_ERR_INVALID_ARGUMENT and enqueue nothing. M <= 8 needs
 * no scratch and has no such limit. Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (several streams, or several
 * host threads) race on it; calls in order on one stream do not. Asynchronous
 * on `stream`.
 */
q2k_status q2k_matmul_noalloc(const float *x, const void *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                              void *stream);

/*
 * q2k_matmul_batched — a batch of independent small products,
 *   y[b][M, N] = x[b][M, K] * W[b][N, K]^T for b = 0 .. batches-1.
 * Page: test q2_k_batched_mv_is_byte_identical_to_independent_dispatches
 * (quantized_matmul_q2_k_batched_mv with (batches, m, n, k); its result must
 * equal, byte for byte, separate single-matrix calls on slice views).
 *   x  device f32 [batches, M, K] row-major; 16-byte aligned.
 *   w  device Q2_K bytes, batches * N * K/256 * 84 long: matrix b follows
 *      matrix b-1, each laid out as for q2k_matmul; 4-byte aligned.
 *   y  device f32 [batches, M, N] row-major; 16-byte aligned.
 *   batches, N >= 1; 1 <= M <= 8 (the fp32 mat-vec path); K as for q2k_matmul.
 * Slice b of y is bit-identical to q2k_matmul(x + b*M*K, w + b*N*K/256*84,
 * y + b*M*N, M, N, K), whatever the other slices hold. Asynchronous on
 * `stream`. Allocates nothing; more than 65535 problems run in several
 * launches.
 */
q2k_status q2k_matmul_batched(const float *x, const void *w, float *y, uint32_t batches, uint32_t M, uint32_t N,
                              uint32_t K, void *stream);

/*
 * Expert-routed product (mixture-of-experts "mm_id").
 * Page: fn run_expert (GgmlQuantizedMatmulIdParams { n_tokens, top_k, n, k,
 * n_experts, expert_stride }; tests q2_k_expert_routed_metal_matches_reference,
 * q2_k_expert_mm_id_top_k_6_matches_reference,
 * q2_k_public_prefill_top_k_6_matches_reference) and test
 * q2_k_slotted_down_mm_is_byte_identical_to_flattened_rows.
 * Route r = token * top_k + slot (0 <= r < n_tokens * top_k) multiplies an
 * activation row by expert e = ids[r]:
 *     y[r, j] = sum_k x[row(r), k] * W_e[j, k],   j < n,
 * with row(r) = r / top_k (x is [n_tokens, k]) or, for the slotted call,
 * row(r) = r (x is [n_tokens, top_k, k]). Expert e's weights are n rows of
 * k/256 Q2_K blocks (layout as for q2k_matmul) starting e * expert_stride
 * bytes into w.
 *   x       device f32, 16-byte aligned.
 *   w       device Q2_K bytes, (n_experts - 1) * expert_stride + n * k/256 * 84
 *           long; 4-byte aligned. Bytes between experts are never read.
 *   ids     device u32 [n_tokens, top_k]; 4-byte aligned; any values.
 *   y       device f32 [n_tokens * top_k, n]; 16-byte aligned.
 *   status  device int or NULL. A route whose id is >= n_experts reads no
 *           weights and gets a row of NaN; if any route does, *status is set
 *           to 1 (never cleared by libq2k). The call itself still returns
 *           Q2K_OK: ids live on the device and are not waited for.
 * Limits: n_tokens, top_k, n >= 1; k a multiple of 256, 256 <= k <= 2^21;
 * 1 <= n_experts <= 512; n_tokens * top_k <= 2^24; expert_stride a multiple
 * of 4 and >= n * k/256 * 84. Outputs may not overlap inputs (or each other).
 * Two schedules compute it:
 *   - fp32 mat-vec per route (Q2K_PATH_GEMV): the M <= 2 bound of q2k_matmul;
 *     route r's row is bit-identical to q2k_matmul(x row, W_e, M = 1).
 *   - matrix-core (Q2K_PATH_MFMA): routes grouped by expert in increasing
 *     route order, bf16(x) * bf16(w) with fp32 accumulation in tiles of up to
 *     128 routes: |y - exact| <= 4e-3 * sum|x*w| + 1e-6. The rows of expert e
 *     are bit-identical to q2k_matmul_path(.., Q2K_PATH_MFMA) of W_e with the
 *     activation rows routed to e, stacked in route order.
 * Asynchronous on `stream`.
 */
typedef struct q2k_matmul_id_params {
    uint32_t n_tokens;      /* tokens, >= 1 */
    uint32_t top_k;         /* routes per token, >= 1 */
    uint32_t n;             /* weight rows per expert = output columns, >= 1 */
    uint32_t k;             /* activation width, a multiple of 256 */
    uint32_t n_experts;     /* 1 .. 512 */
    uint32_t reserved;      /* must be 0 */
    uint64_t expert_stride; /* bytes from one expert's weights to the next */
} q2k_matmul_id_params;

/* q2k_matmul_id — the routed product with libq2k choosing the schedule the way
 * the page's test tolerances do: the matrix-core schedule when n_tokens > 32
 * and top_k is 1, 6 or 8, the fp32 mat-vec otherwise. The matrix-core schedule
 * uses the stream's workspace (conventions above). */
q2k_status q2k_matmul_id(const float *x, const void *w, const uint32_t *ids, float *y,
                         const q2k_matmul_id_params *p, int *status, void *stream);

/* q2k_matmul_id with an explicit schedule (Q2K_PATH_AUTO = q2k_matmul_id). */
q2k_status q2k_matmul_id_path(const float *x, const void *w, const uint32_t *ids, float *y,
                              const q2k_matmul_id_params *p, int *status, q2k_path path, void *stream);

/* Bytes of caller-held scratch the pooled calls need for these parameters
 * (the slotted call needs the same), or 0 if the parameters are invalid. */
uint64_t q2k_matmul_id_scratch_bytes(const q2k_matmul_id_params *p);

/* q2k_matmul_id_pooled — the matrix-core schedule with caller-held scratch
 * (page: quantized_matmul_id_ggml_pooled with IdMmScratch). scratch is device
 * memory of at least q2k_matmul_id_scratch_bytes(p) bytes, 256-byte aligned,
 * not overlapping any argument; its contents on entry do not matter and it
 * is in use until the call's work on `stream` ends. Same result, bit for bit,
 * as q2k_matmul_id_path(.., Q2K_PATH_MFMA, ..). */
q2k_status q2k_matmul_id_pooled(const float *x, const void *w, const uint32_t *ids, float *y,
                                const q2k_matmul_id_params *p, void *scratch, uint64_t scratch_bytes,
                                int *status, void *stream);

/* q2k_matmul_id_pooled_pair — two weight sets with one routing (page:
 * quantized_matmul_id_ggml_pooled_pair, the gate/up projections): y0 from w0
 * and y1 from w1, both laid out as w. The routing, bf16 activations and tile
 * schedule are shared, so each output equals, bit for bit, a pooled call on
 * its own weights (the page's "prepared schedule preserves ordinary mm_id
 * output" check: w0 == w1 gives y0 == y1). y0 and y1 may not overlap. */
q2k_status q2k_matmul_id_pooled_pair(const float *x, const void *w0, const void *w1, const uint32_t *ids,
                                     float *y0, float *y1, const q2k_matmul_id_params *p, void *scratch,
                                     uint64_t scratch_bytes, int *status, void *stream);

/* q2k_matmul_id_pooled_slotted — one activation row per route (page:
 * quantized_matmul_id_ggml_pooled_slotted, the down projection): x is
 * [n_tokens, top_k, k] and y [n_tokens, top_k, n]. Byte-identical to
 * q2k_matmul_id_pooled on the flattened problem (n_tokens * top_k tokens,
 * top_k = 1, the same ids). */
q2k_status q2k_matmul_id_pooled_slotted(const float *x, const void *w, const uint32_t *ids, float *y,
                                        const q2k_matmul_id_params *p, void *scratch, uint64_t scratch_bytes,
                                        int *status, void *stream);

/*
 * q2k_embedding_gather — out[t, :] = decoded row ids[t] of a Q2_K table.
 * Page: test q2_k_embedding_gather_matches_canonical_rows_and_rejects_bad_ids
 * (EmbeddingQ2KParams { vocab_size, embed_dim, n_tokens }; an id equal to
 * vocab must make the call fail).
 *   table     device Q2_K bytes, vocab * embed_dim/256 * 84 long; 4-byte aligned.
 *   ids       device u32 [n_tokens]; 4-byte aligned. Duplicates are allowed.
 *   out       device f32 [n_tokens, embed_dim] row-major; 16-byte aligned.
 *   vocab, n_tokens >= 1; embed_dim >= 256 and a multiple of 256.
 * Rows are bit-identical to q2k_dequantize of the same blocks. The kernel
 * checks every id on the GPU and never reads a row at or beyond vocab; the
 * call then waits for the kernel and returns Q2K_ERR_ID_OUT_OF_RANGE if any id
 * was >= vocab. In that case rows of valid ids hold their values and rows of
 * bad ids are left unwritten. Synchronous: it returns after the kernel, and
 * so all work queued on `stream` before it, has ended. The wait polls a
 * pinned word that a one-thread kernel queued behind the gather writes; past
 * about 2 ms it waits on `stream` instead (which also reports a fault in work
 * queued earlier). Not allowed while `stream` is capturing a graph
 * (Q2K_ERR_INVALID_ARGUMENT; use q2k_embedding_gather_async). Uses one pinned
 * and one device word per device, created on first use; calls from several
 * host threads are serialised on them.
 */
q2k_status q2k_embedding_gather(const void *table, const uint32_t *ids, float *out, uint32_t vocab,
                                uint32_t embed_dim, uint32_t n_tokens, void *stream);

/*
 * q2k_embedding_gather_async — the same gather without the wait, for callers
 * that issue many gathers and check the ids once (a serving loop).
 * Page: the same test as q2k_embedding_gather; the bad id is still rejected,
 * but reported through *status instead of the return value.
 *   table, ids, out, vocab, embed_dim, n_tokens  as for q2k_embedding_gather.
 *   status  device int (or device-mapped host int), 4-byte aligned, not
 *           overlapping the other buffers; required. If any id is >= vocab the
 *           kernel sets *status to 1; libq2k never clears it (the caller zeroes
 *           it before the first call and reads it after the stream has passed
 *           the calls it covers).
 * Rows of valid ids are bit-identical to q2k_embedding_gather's; rows of bad
 * ids are left unwritten. Returns Q2K_OK once the kernel is enqueued
 * (asynchronous on `stream`); argument errors are reported as for
 * q2k_embedding_gather and enqueue nothing. Allocates nothing.
 */
q2k_status q2k_embedding_gather_async(const void *table, const uint32_t *ids, float *out, uint32_t vocab,
                                      uint32_t embed_dim, uint32_t n_tokens, int *status, void *stream);

/*
 * q2k_argmax_candidates — per slot of [n_slots, vocab] f32 logits: the first
 * maximum and the indices within 0.5 of it.
 * Page: docs.rs source page of mlx-native 0.9.5, src/mlx_native/ops/gpu_sample.rs
 * (dispatch_gpu_sample_argmax_candidates: first-max argmax with lower-index
 * tie-break, candidates are logits >= top1 - 0.5f, the count may exceed cap,
 * overflow is set when it does; n_slots, vocab and cap must be > 0).
 *   logits      device f32 [n_slots, vocab] row-major; 4-byte aligned.
 *   top1_idx    device u32 [n_slots]: the lowest index holding the slot's
 *               maximum, scanning left to right with strict '>' (NaN never
 *               wins; a NaN in column 0 is the scan's start and stays the answer).
 *   top1_val    device f32 [n_slots]: that logit.
 *   cand_count  device u32 [n_slots]: how many logits are >= top1_val - 0.5f
 *               (f32 subtraction); may exceed cap; 0 when top1_val is NaN.
 *   overflow    device u32 [n_slots]: 1 if cand_count > cap, else 0.
 *   cand_ids    device u32 [n_slots, cap]: the first min(cand_count, cap)
 *               candidate indices in increasing order; entries past them are
 *               left unwritten.
 * 1 <= vocab <= 2^29. Outputs may not overlap the logits or each other. Uses the stream's
 * workspace (about 530 bytes per 4096 logits; conventions above). Asynchronous on `stream`.
 */
q2k_status q2k_argmax_candidates(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                 uint32_t *top1_idx, float *top1_val, uint32_t *cand_count, uint32_t *overflow,
                                 uint32_t *cand_ids, void *stream);

/* Device scratch q2k_argmax_candidates_pooled needs for n_slots x vocab logits
 * (n_slots >= 1, 1 <= vocab <= 2^29); *bytes is written only on success. */
q2k_status q2k_argmax_candidates_scratch_bytes(uint32_t n_slots, uint32_t vocab, uint64_t *bytes);

/* q2k_argmax_candidates with caller-held scratch and no allocation: scratch is
 * device memory of at least q2k_argmax_candidates_scratch_bytes bytes, 256-byte
 * aligned, not overlapping any other argument, in use until the call's work on
 * `stream` ends. Same results as q2k_argmax_candidates. */
q2k_status q2k_argmax_candidates_pooled(const float *logits, uint32_t n_slots, uint32_t vocab, uint32_t cap,
                                        uint32_t *top1_idx, float *top1_val, uint32_t *cand_count,
                                        uint32_t *overflow, uint32_t *cand_ids, void *scratch,
                                        uint64_t scratch_bytes, void *stream);

/*
 * GGUF tensor directory (host only; no GPU work).
 * Page: test q2_k_gguf_type_10_parses_with_exact_block_size (GgufFile::open,
 * tensor_info(name) -> ggml_type, byte_len): a GGUF v3 file whose one tensor
 * "q2.weight" has one dimension of 256 and type 10 must report type Q2_K and
 * 84 bytes.
 * The file is "GGUF", u32 version (2 or 3), u64 tensor count, u64 metadata
 * count, the metadata (string key, u32 type, value), then per tensor: string
 * name, u32 n_dims, n_dims u64 extents (fastest first), u32 type, u64 offset
 * into the data section, which starts at the next multiple of 32 bytes (or of
 * the u32 metadata value "general.alignment"). Strings are a u64 length and
 * the bytes; integers are little endian.
 * q2k_gguf_open maps the file read-only and indexes the tensor records; every
 * read is bounds-checked, and any malformed or truncated input is
 * Q2K_ERR_INVALID_ARGUMENT with a message. The handle is caller-owned until
 * q2k_gguf_close; pointers from q2k_gguf_tensor_name / q2k_gguf_tensor_data
 * stay valid until then. Handles may be read from several threads at once.
 */
#define Q2K_GGUF_MAX_DIMS 4
#define Q2K_GGML_TYPE_Q2_K 10

typedef struct q2k_gguf q2k_gguf;

typedef struct q2k_gguf_info {
    uint32_t ggml_type;                /* GGML type code (10 = Q2_K) */
    uint32_t n_dims;                   /* 1 .. Q2K_GGUF_MAX_DIMS */
    uint64_t dims[Q2K_GGUF_MAX_DIMS];  /* extents, fastest-varying first; unused ones are 1 */
    uint64_t file_offset;              /* byte offset of the tensor's data in the file */
    uint64_t byte_len;                 /* data bytes; 0 when the type's size is unknown here
                                          (known: F32 = 0, F16 = 1, Q2_K = 10, BF16 = 30) */
} q2k_gguf_info;

q2k_status q2k_gguf_open(const char *path, q2k_gguf **out);
void q2k_gguf_close(q2k_gguf *f); /* NULL is ignored */
uint64_t q2k_gguf_tensor_count(const q2k_gguf *f);
/* Name of tensor `index` in file order, or NULL if out of range. */
const char *q2k_gguf_tensor_name(const q2k_gguf *f, uint64_t index);
/* Unknown name, a row extent that is not a whole number of blocks, or data
 * outside the file: Q2K_ERR_INVALID_ARGUMENT. */
q2k_status q2k_gguf_tensor_info(const q2k_gguf *f, const char *name, q2k_gguf_info *info);
/* Host pointer to the tensor's bytes inside the mapping (for upload with
 * hipMemcpy); fails if the type's size is unknown. */
q2k_status q2k_gguf_tensor_data(const q2k_gguf *f, const char *name, const void **data, uint64_t *byte_len);

/* Static English name of a status code ("Q2K_OK", ...). Never NULL. */
const char *q2k_status_string(q2k_status s);

/* Detail of the last failing call on this host thread (empty string if none).
 * The pointer stays valid until the next libq2k call on the same thread. */
const char *q2k_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* Q2K_H */
