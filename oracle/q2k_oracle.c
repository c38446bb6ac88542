/*
 * Q2_K CPU oracle — TEST INFRASTRUCTURE ONLY.
 *
 * This file is the slow, obviously-correct definition that the HIP path is
 * checked against. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it. The product library never links, calls or
 * falls back to it, and the two share no code, header, table or helper.
 *
 * Source of every rule below: the docs.rs source page of mlx-native 0.10.8,
 * tests/deepseek_q2_k.rs ("GGML Q2_K loading and Metal execution proofs for
 * DeepSeek-V4 Q2_K_S"). Functions cite the item on that page they restate:
 *   - constants QK_K / BLOCK_BYTES and fn block: the 84-byte super-block layout
 *     (16 scale bytes, 64 code bytes, f16 d, f16 dmin);
 *   - fn reference_dequant: decode order and arithmetic;
 *   - fn cpu_dot: the page's f32 dot product;
 *   - test q2_k_host_decode_rejects_malformed_buffers: length checks;
 *   - test q2_k_embedding_gather_matches_canonical_rows_and_rejects_bad_ids:
 *     gather semantics and the id == vocab rejection;
 *   - fn run_dense: y[m, n] = sum_k x[m, k] * w[n, k], rows of w made of
 *     K/256 consecutive blocks;
 *   - fn run_expert and the slotted down-projection test: the expert-routed
 *     product, one expert per (token, slot) route.
 *
 * Precision: the page decodes in f32 (d and dmin widened to f32, products and
 * the final subtraction in f32), so dequantization is done in f32 here too.
 * Matmul accumulates in f64 (every f32*f32 product is exact in f64). Build with
 * -O2 -ffp-contract=off and without fast-math so each f32 operation is one
 * IEEE-754 operation.
 *
 * Parity pins (the tests that tie this file to the page, not to itself):
 * hand-decoded elements of the page's block(5) fixture, an exhaustive f16
 * decode check against numpy, format invariants (all-zero codes, all-three
 * codes, zero scale, zero min, single-bit perturbations), the closed-form
 * element map, brute-force exact-rational matmuls, and torch's bf16 rounding.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK_K 256
#define BLOCK_BYTES 84

/* IEEE-754 binary16 -> binary32, written from the format definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. Exponent 0 is zero
 * or subnormal (fraction * 2^-24); exponent 31 is Inf (fraction 0) or NaN.
 * The page stores d and dmin as little-endian f16 at bytes 80..83 of a block. */
float oracle_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? (double)NAN : (double)INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25);
    }
    return (float)(sign ? -v : v);
}

static float block_d(const uint8_t *blk) {
    return oracle_f16_to_f32((uint16_t)(blk[80] | (blk[81] << 8)));
}

static float block_dmin(const uint8_t *blk) {
    return oracle_f16_to_f32((uint16_t)(blk[82] | (blk[83] << 8)));
}

/* fn reference_dequant (decode rule and output order), walked by sub-block.
 * The 256 weights of a block form 16 sub-blocks of 16 consecutive weights.
 * Sub-block j takes scale byte j (low nibble: the multiplier of d; high
 * nibble: the multiplier of dmin) and its 2-bit codes from the 16 consecutive
 * code bytes that start at qs offset 32*(j/8) + 16*(j%2), all at bit offset
 * 2*((j/2)%4). Taking j = 0, 1, ..., 15 visits the page's order exactly:
 * first half (j < 8) before second, within a half the bit offsets 0, 2, 4, 6,
 * within an offset the lower 16 code bytes before the upper 16. Each weight
 * is (d * sc) * code - dmin * mn in f32, written to out[16 j + i]. */
void oracle_dequant_block(const uint8_t *blk, float *out) {
    const float d = block_d(blk);
    const float dmin = block_dmin(blk);
    for (int j = 0; j < 16; ++j) {
        const uint8_t sub_scale = blk[j];
        const float step = d * (float)(sub_scale & 0x0f);
        const float floor_value = dmin * (float)(sub_scale >> 4);
        const uint8_t *code_bytes = blk + 16 + 32 * (j / 8) + 16 * (j % 2);
        const int bit = 2 * ((j / 2) % 4);
        for (int i = 0; i < 16; ++i) {
            const int code = (code_bytes[i] >> bit) & 3;
            out[16 * j + i] = step * (float)code - floor_value;
        }
    }
}

/* The same decode, addressed per element instead of in loop order: element e
 * lies in half e/128, at 2-bit position (e/32)%4, segment (e/16)%2, lane e%16.
 * So its scale byte is number e/16 and its code byte is 32*(e/128) + e%32.
 * Kept as an independent cross-check of the loop-order decode. */
float oracle_dequant_element(const uint8_t *blk, int e) {
    const uint8_t s = blk[e >> 4];
    const int byte = 32 * (e >> 7) + (e & 31);
    const int shift = 2 * ((e >> 5) & 3);
    const int code = (blk[16 + byte] >> shift) & 3;
    const float dl = block_d(blk) * (float)(s & 0x0f);
    const float ml = block_dmin(blk) * (float)(s >> 4);
    return dl * (float)code - ml;
}

/* test q2_k_host_decode_rejects_malformed_buffers: a byte length that is not a
 * whole number of 84-byte blocks, or an output that is not exactly 256 values
 * per block, is an error. Returns 0 on success, -1 on a rejected length. */
int oracle_dequantize(const uint8_t *bytes, size_t nbytes, float *out, size_t out_elems) {
    if (nbytes == 0 || nbytes % BLOCK_BYTES != 0) return -1;
    const size_t nblocks = nbytes / BLOCK_BYTES;
    if (out_elems != nblocks * QK_K) return -1;
    for (size_t b = 0; b < nblocks; ++b)
        oracle_dequant_block(bytes + b * BLOCK_BYTES, out + b * QK_K);
    return 0;
}

/* Round an f32 to the nearest bf16 (8-bit significand), ties to even, returned
 * widened back to f32. NaN stays NaN. Written from the format definition: keep
 * the top 16 bits, adding half an ulp plus the parity of the kept lsb. */
float oracle_bf16_round(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
        u |= 0x00400000u; /* quiet NaN */
        u &= 0xffff0000u;
    } else {
        const uint32_t lsb = (u >> 16) & 1u;
        u = (u + 0x7fffu + lsb) & 0xffff0000u;
    }
    float r;
    memcpy(&r, &u, 4);
    return r;
}

static int matmul_shape_ok(long M, long N, long K) {
    return M > 0 && N > 0 && K > 0 && K % QK_K == 0;
}

/* Dequantize row n of w (K/256 consecutive blocks) into wrow[K]. */
static void dequant_row(const uint8_t *w, long n, long K, float *wrow) {
    const long nb = K / QK_K;
    const uint8_t *row = w + (size_t)n * (size_t)nb * BLOCK_BYTES;
    for (long b = 0; b < nb; ++b)
        oracle_dequant_block(row + (size_t)b * BLOCK_BYTES, wrow + b * QK_K);
}

/* fn run_dense: y[m, n] = sum over k of x[m, k] * w[n, k], with x row-major
 * [M, K] f32, w N rows of K/256 blocks, y row-major [M, N]. Accumulates in f64
 * in increasing k; also returns a[m, n] = sum over k of |x[m, k] * w[n, k]|,
 * the scale the tolerances are stated against. bf16_operands = 1 first rounds
 * both operands to bf16 (ties to even), the operand precision of the matrix-
 * core path. One thread computes each output, so results do not depend on
 * nthreads. Returns 0, or -1 for a rejected shape. */
int oracle_matmul(const float *x, const uint8_t *w, double *y, double *a,
                  long M, long N, long K, int bf16_operands, int nthreads) {
    if (!matmul_shape_ok(M, N, K)) return -1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)K);
        float *xrow = (float *)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
        for (long n = 0; n < N; ++n) {
            dequant_row(w, n, K, wrow);
            if (bf16_operands)
                for (long k = 0; k < K; ++k) wrow[k] = oracle_bf16_round(wrow[k]);
            for (long m = 0; m < M; ++m) {
                const float *xm = x + (size_t)m * (size_t)K;
                if (bf16_operands) {
                    for (long k = 0; k < K; ++k) xrow[k] = oracle_bf16_round(xm[k]);
                    xm = xrow;
                }
                double s = 0.0, sa = 0.0;
                for (long k = 0; k < K; ++k) {
                    const double p = (double)xm[k] * (double)wrow[k];
                    s += p;
                    sa += fabs(p);
                }
                y[(size_t)m * (size_t)N + (size_t)n] = s;
                if (a) a[(size_t)m * (size_t)N + (size_t)n] = sa;
            }
        }
        free(wrow);
        free(xrow);
    }
    return 0;
}

/* fn cpu_dot: f32 products summed left to right in f32, as the page's test
 * computes its expected dense outputs. Same shapes as oracle_matmul. */
int oracle_matmul_f32seq(const float *x, const uint8_t *w, float *y, long M, long N, long K) {
    if (!matmul_shape_ok(M, N, K)) return -1;
    float *wrow = (float *)malloc(sizeof(float) * (size_t)K);
    for (long n = 0; n < N; ++n) {
        dequant_row(w, n, K, wrow);
        for (long m = 0; m < M; ++m) {
            const float *xm = x + (size_t)m * (size_t)K;
            float s = 0.0f;
            for (long k = 0; k < K; ++k) s += wrow[k] * xm[k];
            y[(size_t)m * (size_t)N + (size_t)n] = s;
        }
    }
    free(wrow);
    return 0;
}

/* test q2_k_embedding_gather_matches_canonical_rows_and_rejects_bad_ids:
 * out[t, :] is the decoded table row ids[t]; the table is [vocab, embed_dim]
 * weights stored as embed_dim/256 blocks per row. Any id >= vocab (the page
 * tries id == vocab) is an error, detected before anything is written.
 * Returns 0, -1 for a rejected shape, -2 for an out-of-range id. */
int oracle_gather(const uint8_t *table, const uint32_t *ids, float *out,
                  long vocab, long embed_dim, long n_tokens, int nthreads) {
    if (vocab <= 0 || embed_dim <= 0 || n_tokens <= 0 || embed_dim % QK_K != 0) return -1;
    for (long t = 0; t < n_tokens; ++t)
        if ((long)ids[t] >= vocab) return -2;
    if (nthreads < 1) nthreads = 1;
    const long nb = embed_dim / QK_K;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (long t = 0; t < n_tokens; ++t) {
        const uint8_t *row = table + (size_t)ids[t] * (size_t)nb * BLOCK_BYTES;
        float *o = out + (size_t)t * (size_t)embed_dim;
        for (long b = 0; b < nb; ++b)
            oracle_dequant_block(row + (size_t)b * BLOCK_BYTES, o + b * QK_K);
    }
    return 0;
}

/* docs.rs source page of mlx-native 0.9.5, src/mlx_native/ops/gpu_sample.rs
 * (dispatch_gpu_sample_argmax_candidates and its module comment): per slot of
 * [n_slots, vocab] f32 logits, the first maximum found by a left-to-right scan
 * with strict '>' (lower index wins ties; NaN never compares greater, so a
 * NaN in column 0 stays the answer), the count of logits >= top1 - 0.5f
 * (computed in f32), an overflow flag when that count exceeds cap, and the
 * first min(count, cap) candidate indices in increasing order (entries past
 * them are not written). Returns 0, or -1 for a zero size. */
int oracle_argmax_candidates(const float *logits, long n_slots, long vocab, long cap,
                             uint32_t *top1_idx, float *top1_val, uint32_t *cand_count,
                             uint32_t *overflow, uint32_t *cand_ids) {
    if (n_slots <= 0 || vocab <= 0 || cap <= 0) return -1;
    for (long s = 0; s < n_slots; ++s) {
        const float *row = logits + (size_t)s * (size_t)vocab;
        long best = 0;
        for (long i = 1; i < vocab; ++i)
            if (row[i] > row[best]) best = i;
        const float top = row[best];
        const float thr = top - 0.5f;
        uint32_t n = 0;
        for (long i = 0; i < vocab; ++i) {
            if (row[i] >= thr) {
                if ((long)n < cap) cand_ids[(size_t)s * (size_t)cap + n] = (uint32_t)i;
                ++n;
            }
        }
        top1_idx[s] = (uint32_t)best;
        top1_val[s] = top;
        cand_count[s] = n;
        overflow[s] = (long)n > cap ? 1u : 0u;
    }
    return 0;
}

/* Expert-routed product of the Q2_K page (fn run_expert, and the slotted
 * test q2_k_slotted_down_mm_is_byte_identical_to_flattened_rows): route
 * r = token * top_k + slot multiplies by expert ids[r]. Its output row is
 * out[r, row] = sum over k of x[xr, k] * W_e[row, k], where xr = r / top_k
 * (one activation row per token) or xr = r when `slotted` (one activation row
 * per route, input [tokens, top_k, K]). Expert e's weights start
 * e * expert_stride bytes into w and hold n rows of K/256 blocks each. The
 * page states no rule for an id >= n_experts; here such a route's outputs are
 * all NaN (never a read outside w) and it is counted in *bad. Accumulates in
 * f64 in increasing k and returns a = sum |x * w| beside y, like
 * oracle_matmul; bf16_operands rounds both operands to bf16 first. Returns 0,
 * or -1 for a rejected shape. */
int oracle_matmul_id(const float *x, const uint8_t *w, const uint32_t *ids, double *y, double *a,
                     long n_tokens, long top_k, long n, long K, long n_experts, long expert_stride,
                     int slotted, int bf16_operands, int nthreads, long *bad) {
    if (n_tokens <= 0 || top_k <= 0 || n <= 0 || n_experts <= 0 || !matmul_shape_ok(1, n, K)) return -1;
    if (expert_stride < n * (K / QK_K) * BLOCK_BYTES) return -1;
    if (nthreads < 1) nthreads = 1;
    const long routes = n_tokens * top_k;
    long nbad = 0;
    for (long r = 0; r < routes; ++r)
        if ((long)ids[r] >= n_experts) ++nbad;
    if (bad) *bad = nbad;
#pragma omp parallel num_threads(nthreads)
    {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)K);
        float *xrow = (float *)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
        for (long r = 0; r < routes; ++r) {
            double *yr = y + (size_t)r * (size_t)n;
            double *ar = a ? a + (size_t)r * (size_t)n : NULL;
            const long e = (long)ids[r];
            if (e >= n_experts) {
                for (long row = 0; row < n; ++row) {
                    yr[row] = NAN;
                    if (ar) ar[row] = NAN;
                }
                continue;
            }
            const long xr = slotted ? r : r / top_k;
            const float *xm = x + (size_t)xr * (size_t)K;
            for (long k = 0; k < K; ++k) xrow[k] = bf16_operands ? oracle_bf16_round(xm[k]) : xm[k];
            const uint8_t *we = w + (size_t)e * (size_t)expert_stride;
            for (long row = 0; row < n; ++row) {
                dequant_row(we, row, K, wrow);
                double s = 0.0, sa = 0.0;
                for (long k = 0; k < K; ++k) {
                    const float wk = bf16_operands ? oracle_bf16_round(wrow[k]) : wrow[k];
                    const double p = (double)xrow[k] * (double)wk;
                    s += p;
                    sa += fabs(p);
                }
                yr[row] = s;
                if (ar) ar[row] = sa;
            }
        }
        free(wrow);
        free(xrow);
    }
    return 0;
}
