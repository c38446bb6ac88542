// HIP kernels of the Q2_K weight path for gfx950 (MI355X).
//
// Block format and decode rule: docs.rs source page of mlx-native 0.10.8,
// tests/deepseek_q2_k.rs (constants QK_K / BLOCK_BYTES, fn block,
// fn reference_dequant). An 84-byte super-block holds 256 weights: 16 scale
// bytes (low nibble sc, high nibble mn), 64 code bytes (four 2-bit codes
// each), f16 d at byte 80 and f16 dmin at byte 82. Weight e has scale byte
// e/16 and code (qs[32*(e/128) + e%32] >> 2*((e/32)%4)) & 3, and equals
// f32(d)*sc*q - f32(dmin)*mn. Because d*sc*q and dmin*mn are exact in f32, the
// value has one correct f32 rounding; the kernels reproduce it bit for bit.
//
// Built with -ffp-contract=off: every FMA below is written as one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "q2k_launch.h"

namespace q2k {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr uint32_t kWave = 64;

// d (bytes 80..81) and dmin (bytes 82..83) arrive together as one dword.
__device__ __forceinline__ float f16_low(uint32_t v) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v & 0xffffu)));
}
__device__ __forceinline__ float f16_high(uint32_t v) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v >> 16)));
}

__device__ __forceinline__ uint32_t load_u32(const uint8_t *p) {
    return *reinterpret_cast<const uint32_t *>(p);
}

// Raw buffer resources (gfx9 dword 3): loads past num_records return zero,
// which is how lanes beyond the end of the data read nothing.
constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRsrcFlags);
}

// Weights e0..e0+3 (e0 % 4 == 0) of one block. The four share a scale byte and
// one 2-bit position of four consecutive code bytes.
__device__ __forceinline__ float4 decode_quad(const uint8_t *blk, uint32_t e0) {
    const uint32_t sbyte = blk[e0 >> 4];
    const uint32_t codes = load_u32(blk + 16 + 32 * (e0 >> 7) + (e0 & 31));
    const uint32_t dd = load_u32(blk + 80);
    const float dl = f16_low(dd) * static_cast<float>(sbyte & 15u);
    const float ml = f16_high(dd) * static_cast<float>(sbyte >> 4);
    const uint32_t c = (codes >> (2 * ((e0 >> 5) & 3))) & 0x03030303u;
    float4 r;
    r.x = dl * static_cast<float>(c & 0xffu) - ml;
    r.y = dl * static_cast<float>((c >> 8) & 0xffu) - ml;
    r.z = dl * static_cast<float>((c >> 16) & 0xffu) - ml;
    r.w = dl * static_cast<float>(c >> 24) - ml;
    return r;
}

// ---------------------------------------------------------------------------
// Dequantize and gather share one shape: a wavefront decodes a run of
// consecutive blocks. It first copies their bytes into its own LDS region
// with direct buffer-to-LDS dword loads, all in flight at once, then writes
// block i as one 1 KiB run of 16-byte stores, lane l taking weights
// 4l..4l+3. With one block per wavefront (84 bytes of reads in flight) the
// dequantize mostly waited on memory latency; with runs of 32 blocks a
// wavefront's whole input (2688 bytes) is requested before any of it is
// needed (65536 blocks: 12.2 us, against 12.3-12.5 us with runs of 64 and
// 12.7 us with runs of 16). A wavefront only touches its own region, so
// there are no barriers.
constexpr uint32_t kRunBlocks = 32;  // blocks per dequantize wavefront
// Its region: 672 dwords of blocks, rounded up to whole loads of 64 dwords (the
// last load reads past the run, beyond the descriptor: zeros).
constexpr uint32_t kRunDwords = (kRunBlocks * kBlockBytes / 4 + kWave - 1) / kWave * kWave;

// Copies blocks src[0 .. nb) into r (ceil(21 nb / 64) * 64 dwords, which r
// must hold) and waits until they are in. Loads past the last block lie
// beyond the descriptor and read zeros.
__device__ __forceinline__ void stage_blocks(const uint8_t *src, uint32_t nb, uint32_t *r, uint32_t lane) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, nb * kBlockBytes);
    const uint32_t loads = (nb * (kBlockBytes / 4) + kWave - 1) / kWave;
    for (uint32_t j = 0; j < loads; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(r + kWave * j), 4,
                                                 static_cast<int>(4u * (kWave * j + lane)), 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront wrote the whole region
}

__global__ __launch_bounds__(256) void k_dequantize(const uint8_t *__restrict__ blocks, float4 *__restrict__ out,
                                                    uint64_t nblocks) {
    __shared__ __attribute__((aligned(16))) uint32_t raw[4][kRunDwords];
    const uint32_t lane = threadIdx.x & (kWave - 1u);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint64_t b0 = (static_cast<uint64_t>(blockIdx.x) * 4u + wave) * kRunBlocks;
    if (b0 >= nblocks) return;
    const uint32_t nb = static_cast<uint32_t>(min(static_cast<uint64_t>(kRunBlocks), nblocks - b0));
    stage_blocks(blocks + b0 * kBlockBytes, nb, raw[wave], lane);
    const uint8_t *rb = reinterpret_cast<const uint8_t *>(raw[wave]);
    for (uint32_t i = 0; i < nb; ++i) out[(b0 + i) * 64u + lane] = decode_quad(rb + i * kBlockBytes, 4u * lane);
}

// Embedding gather: wavefront u takes run u % runs of token u / runs, where a
// row of blocks_per_row blocks splits into runs = ceil(blocks_per_row / 2)
// runs of 2 blocks. A gather moves few bytes per row, so short runs keep more
// wavefronts busy (512 rows of 16 blocks, back to back: 3.68 us with 2-block
// runs, 3.76 us with 4, 3.85 us with 1, 3.88 us with 8; 5.3 us with 64 in an
// earlier form). A token whose id is >= vocab raises the status word and its
// row is neither read nor written.
constexpr uint32_t kGatherRun = 2;
constexpr uint32_t kGatherDwords = (kGatherRun * kBlockBytes / 4 + kWave - 1) / kWave * kWave;

__global__ __launch_bounds__(256) void k_gather(const uint8_t *__restrict__ table, const uint32_t *__restrict__ ids,
                                                float4 *__restrict__ out, uint32_t vocab, uint32_t blocks_per_row,
                                                uint32_t n_tokens, int *status, int bad_value) {
    __shared__ __attribute__((aligned(16))) uint32_t raw[4][kGatherDwords];
    const uint32_t lane = threadIdx.x & (kWave - 1u);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t runs = (blocks_per_row + kGatherRun - 1) / kGatherRun;
    const uint64_t u = static_cast<uint64_t>(blockIdx.x) * 4u + wave;
    if (u >= static_cast<uint64_t>(n_tokens) * runs) return;
    const uint32_t t = static_cast<uint32_t>(u / runs), c = static_cast<uint32_t>(u % runs);
    const uint32_t id = ids[t];
    if (id >= vocab) {
        if (c == 0 && lane == 0) __hip_atomic_store(status, bad_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        return;
    }
    const uint32_t kb0 = c * kGatherRun, nb = min(kGatherRun, blocks_per_row - kb0);
    const uint64_t row_bytes = static_cast<uint64_t>(blocks_per_row) * kBlockBytes;
    stage_blocks(table + id * row_bytes + kb0 * kBlockBytes, nb, raw[wave], lane);
    const uint8_t *rb = reinterpret_cast<const uint8_t *>(raw[wave]);
    float4 *orow = out + (static_cast<uint64_t>(t) * blocks_per_row + kb0) * 64u;
    for (uint32_t i = 0; i < nb; ++i) orow[i * 64u + lane] = decode_quad(rb + i * kBlockBytes, 4u * lane);
}

// The end of a synchronous gather, for a host that polls memory instead of
// synchronizing the stream (which costs several microseconds more): this
// kernel starts only after the gather kernel before it on the stream has
// ended, and its one store to host-visible memory carries both the call's
// sequence number and whether that gather saw a bad id (the gather stores the
// number itself into *status, so a value left by an earlier call never reads
// as this call's). It clears *status before that store (release order), so a
// marker does not outlive its call and cannot meet a reused sequence number
// after the numbers wrap. Folding this into the gather (the last workgroup
// to finish publishing) costs more: every workgroup then needs an
// agent-scope release, an L2 write-back, before it counts itself.
__global__ __launch_bounds__(64) void k_gather_done(int *__restrict__ status, int seq, int *host_word) {
    if (threadIdx.x != 0) return;
    const int v = __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (v != 0) __hip_atomic_store(status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(host_word, (seq << 2) | 2 | (v == seq ? 1 : 0), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (DPP, gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Batched GEMV: grid.y walks independent problems laid out batch-major;
// problem b reads x + b * x_elems and w + b * w_bytes and writes y + b * y_elems.
// Every problem runs exactly the instructions of a single call, so a batched
// result is bit-identical to separate calls on the same slices.
struct GemvBatch {
    uint64_t x_elems, w_bytes, y_elems;
};

// Expert-routed GEMV: grid.y walks routes route0 ..; route r multiplies
// activation row r / x_div by expert ids[r] (expert_stride bytes apart) into
// output row r. A route whose id is >= n_experts reads nothing, writes NaN to
// its row and raises *status (when status is not null).
struct GemvRoute {
    const uint32_t *ids;
    int *status;
    uint64_t expert_stride;
    uint32_t route0, x_div, n_experts;
};

// ---------------------------------------------------------------------------
// fp32 GEMV for M <= 2 (decode).
//
// A workgroup of 16 / BW wavefronts owns (16 / BW) * NI consecutive weight
// rows, taken 16 / BW at a time (a row group; NI of them), and walks K in
// chunks of 16 blocks (4096 weights). Wavefront w covers blocks BW w ..
// BW w + BW - 1 of a chunk; lane l of it works on row l / (4 BW) of the
// current group, block (l / 4) % BW of the wavefront's BW and code segment
// g = l % 4: the 16 code bytes qs[32h + 16s ..] with h = g / 2, s = g % 2, at
// all four 2-bit positions p -- that is, all of sub-blocks 8h + 2p + s (64
// weights). The lane's 64 activations depend only on (block, segment): each
// wavefront copies its blocks' activations into LDS once per chunk, and each
// lane reads its 64 from there into registers, where they stay for all the
// workgroup's rows. All of a chunk's loads are issued before any arithmetic,
// so the workgroup's whole share of the matrix is in flight at once.
//
// The lane's arithmetic per row is segment_value (below): T = sum q*x per
// sub-block, then d * (sum sc * T) - dmin * (sum mn * S), S = sum x over the
// sub-block. The four lanes of a (block, segment) hold the same activations,
// so each computes one of their four sums S (pairwise) and they meet in LDS.
// Partial sums are reduced over the 4 BW lanes of a row with DPP and over the
// wavefronts through LDS, in a fixed order: the four segments of a block
// pairwise, then blocks pairwise up to four, then the four quarters of the
// chunk left to right, so both shapes below give bit-identical rows.
//
// Error bound (first order, u = 2^-24): every term of the result passes
// through at most 16 roundings in T (the first FMA adds to +0), 4 in the sc
// sum, 1 each in the FMAs with d and dmin, 2 per further K chunk of 4096 in
// the running sum and 7 in the reduction over blocks and wavefronts; the min
// terms through fewer. So
//   |y - exact| <= (27 + 2 * ceil(K / 4096)) u * B,
//   B = sum_k |x[k]| * (|d * sc * q| + |dmin * mn|),
// as long as the scaled sums T (q x times 4^p 2^-24) stay in f32's normal range
// (activations above about 2^-100 where they meet non-zero codes). B equals
// sum_k |x * w| unless a block's code and min terms cancel; the 1e-5 * sum|x w|
// rule holds whenever B is within 5.5x of sum |x w| (K <= 4096).
//
// Two shapes. A decode-sized matrix (N = 4096) runs 8 wavefronts of two
// blocks per workgroup and two row groups of 8 (16 rows: 256 workgroups, one
// per CU): twice the wavefronts of the four-block form issue a chunk's loads
// sooner, with the same activation traffic (M = 1: 3.74 us against 3.87 us).
// Once a launch would need more than about one and a half rounds of the
// small shape's resident workgroups (seg_iters_large), the memory system is busy
// anyway and per-lane setup (activations, sub-block sums, reduction) is what
// to amortize: 4 wavefronts of four blocks and eight
// row groups of 4 (32 rows; M = 1, N = 16384: 7.5 us against 8.4 us in the
// small shape's layout). Eight groups measured best for both M (M = 1: 6, 10,
// 12 and 16 slower by 0-15 %; M = 2: 248 VGPRs, two wavefronts per SIMD, and
// still 4-7 % faster than six). A row's arithmetic does not depend on the
// shape.
constexpr uint32_t kSegSmallBW = 2;
constexpr int kSegSmallNI = 2;
constexpr uint32_t kSegLargeBW = 4;
constexpr int kSegLargeNI = 8;
constexpr uint32_t seg_rows(uint32_t bw, int ni) { return 16 / bw * static_cast<uint32_t>(ni); }
static_assert(seg_rows(kSegLargeBW, kSegLargeNI) * (kMaxK / 256) * 84 < (1ull << 31) &&
                  seg_rows(kSegSmallBW, kSegSmallNI) * (kMaxK / 256) * 84 < (1ull << 31),
              "a workgroup's rows fit a 31-bit offset");

// Bytes 0, 1 (W = false) or 2, 3 (W = true) of v, each below 16, as exact integers.
template <bool W>
__device__ __forceinline__ void nibbles2(uint32_t v, float *a, float *b) {
    const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(static_cast<int>(v), 512.0f, W);
    *a = r[0];
    *b = r[1];
}

// acc + f16(half H of codes) * x in one v_fma_mix_f32 (the f16 widening is
// exact, so this is fma(f32(code), x, acc)); written out so that every code
// meets every activation row through this one instruction.
template <int H>
__device__ __forceinline__ float fma_code(uint32_t codes, float x, float acc) {
    float r;
    if constexpr (H == 1)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(codes), "v"(x), "v"(acc));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(codes), "v"(x), "v"(acc));
    return r;
}

struct SegLoads {
    uint32_t q[4];   // the 16 code bytes of the segment
    uint32_t sc[2];  // the 8 scale bytes of the segment's half
    uint32_t dd;     // d, dmin
};

__device__ __forceinline__ SegLoads load_seg(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t g, uint32_t h) {
    SegLoads t;
    const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 + 16 * g, 0, 0);
    const auto sc = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 8 * h, 0, 0);
    t.dd = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 80, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) t.q[j] = q[j];
    t.sc[0] = sc[0];
    t.sc[1] = sc[1];
    return t;
}

// One lane's share of one weight row: the 64 weights of its code segment
// (sub-blocks 8h + 2p + s, p = 0..3, of one block) against its activations
// xv[m][p][i] (element i of sub-block p) and their sums xs[m][p], added to
// acc[m] as acc + d * (sum_p sc_p T_p) - dmin * (sum_p mn_p S_p), T_p = sum_i q x.
// Both M <= 2 kernels use exactly this arithmetic, so a row comes out
// bit-identical from either. scsel picks the lane's four scale bytes.
//
// Codes never pass through a conversion instruction: masked in place within a
// 16-bit half (0x0003 << 2p), a code is the f16 subnormal q * 4^p * 2^-24,
// which v_fma_mix_f32 multiplies by an f32 activation exactly (the odd code
// bytes reach the low byte of a half by one 8-bit shift). T_p is thus carried
// scaled by 4^p 2^-24, and the scale nibbles, converted with the power-of-two
// scales 2^33 and 2^29 (times 4^-1 for positions 1 and 3), carry it back
// exactly.
template <int M>
__device__ __forceinline__ void segment_value(const SegLoads &L, const float (&xv)[M][4][16],
                                              const float (&xs)[M][4], uint32_t scsel, float (&acc)[M]) {
    float t[M][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // One code dword at a time: left free, the scheduler may mask all 16 dwords' codes up front and
        // hold them in 32 registers.
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t v = L.q[j], u = v >> 8;  // u: the odd bytes in the low byte of each half
        uint32_t me[4], mo[4];                  // bytes 4j, 4j+2 and 4j+1, 4j+3 of the segment
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t mask = 0x00030003u << (2 * p);
            me[p] = v & mask;
            mo[p] = u & mask;
        }
        // The four chains (one per position) advance in turn: a chain's next
        // FMA never directly follows its last, so no wait state sits between.
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float a[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) a[p] = fma_code<0>(me[p], xv[m][p][4 * j], j == 0 ? 0.0f : t[m][p]);
#pragma unroll
            for (int p = 0; p < 4; ++p) a[p] = fma_code<0>(mo[p], xv[m][p][4 * j + 1], a[p]);
#pragma unroll
            for (int p = 0; p < 4; ++p) a[p] = fma_code<1>(me[p], xv[m][p][4 * j + 2], a[p]);
#pragma unroll
            for (int p = 0; p < 4; ++p) t[m][p] = fma_code<1>(mo[p], xv[m][p][4 * j + 3], a[p]);
        }
    }
    // Scale bytes 8h + 2p + s (p = 0..3): bytes s, 2 + s of the half's two scale dwords, gathered into one
    // dword; low nibbles sc, high nibbles mn.
    const uint32_t sb = __builtin_amdgcn_perm(L.sc[1], L.sc[0], scsel);
    const uint32_t lo = sb & 0x0F0F0F0Fu, hi = (sb >> 4) & 0x0F0F0F0Fu;
    const auto s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(static_cast<int>(lo), 8589934592.0f, false);  // sc 2^24
    const auto s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(static_cast<int>(lo), 536870912.0f, true);   // sc 2^20
    const float sc[4] = {s01[0], s01[1] * 0.25f, s23[0], s23[1] * 0.25f};  // sc_p 2^(24 - 2p)
    float mn[4];
    nibbles2<false>(hi, &mn[0], &mn[1]);
    nibbles2<true>(hi, &mn[2], &mn[3]);
    const float d = f16_low(L.dd), dmin = f16_high(L.dd);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float codes = sc[0] * t[m][0];
#pragma unroll
        for (int p = 1; p < 4; ++p) codes = __builtin_fmaf(sc[p], t[m][p], codes);
        float mins = mn[0] * xs[m][0];
#pragma unroll
        for (int p = 1; p < 4; ++p) mins = __builtin_fmaf(mn[p], xs[m][p], mins);
        const float a = __builtin_fmaf(d, codes, acc[m]);
        acc[m] = __builtin_fmaf(-dmin, mins, a);
    }
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Wait until at most N vector-memory operations of this wavefront are still in
// flight (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, the other counters at
// their "no wait" maxima).
template <uint32_t N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N < 64, "vmcnt has six bits");
    __builtin_amdgcn_s_waitcnt(static_cast<int>((N & 15u) | ((N >> 4) << 14) | 0x0F70u));
}

// vm_wait<n> for a count known only after unrolling (n <= Hi): the chain of
// comparisons folds to the one wait.
template <uint32_t Hi>
__device__ __forceinline__ void vm_wait_n(uint32_t n) {
    if constexpr (Hi == 0) {
        vm_wait<0>();
    } else {
        if (n >= Hi) vm_wait<Hi>();
        else vm_wait_n<Hi - 1>(n);
    }
}

template <int M, uint32_t BW, int NI, bool kRouted>
__global__ __launch_bounds__(64 * 16 / BW) void k_gemv_seg(const float *__restrict__ x, const uint8_t *__restrict__ w,
                                                float *__restrict__ y, uint32_t N, uint32_t K, GemvBatch bt,
                                                GemvRoute rt) {
    static_assert(BW == 2 || BW == 4, "two or four blocks per wavefront");
    constexpr uint32_t kWaves = 16 / BW, kGroupRows = 16 / BW;
    constexpr uint32_t kRows = kGroupRows * NI;  // rows of the workgroup
    __shared__ float red[kWaves][kRows * M];     // per wavefront: its blocks' sum of each row
    // Per wavefront: x of its BW blocks, block j at float 260 j so that the lanes' 16-byte reads of
    // different blocks fall in different bank groups.
    constexpr uint32_t kXB = 260;
    __shared__ __attribute__((aligned(16))) float xl[kWaves][M][BW * kXB];
    __shared__ __attribute__((aligned(16))) float xsum[kWaves][M][16 * BW];  // per wavefront: S of its sub-blocks
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1);
    const uint32_t row0 = blockIdx.x * kRows;
    if constexpr (kRouted) {
        static_assert(M == 1, "routes are single activation rows");
        const uint32_t r = rt.route0 + blockIdx.y;
        const uint32_t e = rt.ids[r];
        y += static_cast<uint64_t>(r) * N;
        if (e >= rt.n_experts) {
            if (tid < kRows && row0 + tid < N) y[row0 + tid] = __builtin_nanf("");
            if (tid == 0 && rt.status) __hip_atomic_store(rt.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            return;
        }
        x += static_cast<uint64_t>(r / rt.x_div) * K;
        w += e * rt.expert_stride;
    } else {
        x += blockIdx.y * bt.x_elems;
        w += blockIdx.y * bt.w_bytes;
        y += blockIdx.y * bt.y_elems;
    }
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t rr = lane / (4 * BW), bq = (lane >> 2) & (BW - 1), g = lane & 3u, h = g >> 1, s = g & 1u;
    const uint32_t scsel = 0x06040200u + 0x01010101u * s;  // scale bytes s, 2 + s of each scale dword
    const uint32_t nb = K >> 8;
    const uint32_t row_bytes = nb * kBlockBytes;

    // One descriptor spans the workgroup's rows; a lane addresses its row with
    // a 32-bit offset (rows past N reread row N-1 and are never stored). The
    // host guarantees kRows * row_bytes < 2^31.
    const uint32_t nrows = min(kRows, N - row0);
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(w + static_cast<uint64_t>(row0) * row_bytes, nrows * row_bytes);
    uint32_t wrow[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) wrow[i] = min(kGroupRows * i + rr, nrows - 1) * row_bytes;
    __amdgpu_buffer_rsrc_t xr[M];
#pragma unroll
    for (int m = 0; m < M; ++m) xr[m] = buffer_rsrc(x + static_cast<uint64_t>(m) * K, K * 4u);

    float acc[NI][M];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[i][m] = 0.0f;

    for (uint32_t kb0 = 0; kb0 < nb; kb0 += 16) {
        const uint32_t kb = kb0 + BW * wave + bq;
        // Lanes past the end of K aim every weight load beyond the descriptor
        // (they read zeros) and their activation loads beyond K (zeros too).
        const uint32_t boff = kb < nb ? kb * kBlockBytes : 0x80000000u;

        // The wavefront's activations (its BW blocks: 1 KiB each per row of x)
        // go to its own LDS region by direct buffer-to-LDS loads, then each row
        // group's weights are requested in the order they are used. The lanes
        // of a (block, segment), one per row of the group, read the same
        // activations, so loading them once into LDS instead of once per lane
        // keeps most of the activation bytes off the vector-memory path, ahead
        // of the weights.
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (uint32_t j = 0; j < BW; ++j) {
                const uint32_t u = __builtin_amdgcn_readfirstlane(4u * (kb0 + BW * wave) * 256u + 1024u * j);
                // (A descriptor held in a local: this compiler drops the host-side
                // kernel stub when the LDS load takes an element of xr.)
                const __amdgpu_buffer_rsrc_t xm = xr[m];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xm, (__attribute__((address_space(3))) void *)(xl[wave][m] + kXB * j), 16,
                    static_cast<int>(u + 16u * lane), 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
        SegLoads wl[NI];
#pragma unroll
        for (int it = 0; it < NI; ++it) wl[it] = load_seg(wrs, wrow[it] + boff, g, h);
        __builtin_amdgcn_sched_barrier(0);
        // Loads complete in issue order: the activations are in once at most the
        // 3 NI weight loads are still in flight.
        vm_wait<3u * NI>();
        __builtin_amdgcn_sched_barrier(0);
        float xv[M][4][16], xs[M][4];
        // S of sub-block 8h + 2p + s for p = rr % 4: one of the four sums the lane's (block, segment)
        // needs, summed pairwise in element order, then exchanged through LDS ([bq][g][p]; with two
        // blocks per wavefront rows rr and rr + 4 compute, and store, the same sum).
        const uint32_t pq = rr & 3u;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4v t4 = *reinterpret_cast<const f32x4v *>(xl[wave][m] + bq * kXB + 128u * h + 16u * s +
                                                                   32u * pq + 4u * i);
#pragma unroll
                for (int c = 0; c < 4; ++c) v[4 * i + c] = t4[c];
            }
            float s2[8], s4[4];
#pragma unroll
            for (int i = 0; i < 8; ++i) s2[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[i] = s2[2 * i] + s2[2 * i + 1];
            xsum[wave][m][16u * bq + 4u * g + pq] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4v v = *reinterpret_cast<const f32x4v *>(xl[wave][m] + bq * kXB + 128u * h + 16u * s +
                                                                      32u * p + 4u * i);
#pragma unroll
                    for (int c = 0; c < 4; ++c) xv[m][p][4 * i + c] = v[c];
                }
        // The sums were written by other lanes of this wavefront; its LDS operations complete in order.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const f32x4v t4 = *reinterpret_cast<const f32x4v *>(&xsum[wave][m][16u * bq + 4u * g]);
#pragma unroll
            for (int p = 0; p < 4; ++p) xs[m][p] = t4[p];
        }
        // Keep the scheduler from sinking these loads towards their uses.
        __builtin_amdgcn_sched_barrier(0);

        // One row group at a time, in load order: a group's arithmetic waits
        // only for its own loads.
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            __builtin_amdgcn_sched_barrier(0);
            segment_value<M>(wl[it], xv, xs, scsel, acc[it]);
        }
    }

    // Reduction in the association both M <= 2 kernels share: per block the four segments
    // (g0 + g1) + (g2 + g3) (two quad steps), then blocks pairwise: (b0 + b1) by a row_ror:4 step,
    // (b0 + b1) + (b2 + b3) by a row_ror:8 step with four blocks per wavefront (the last lane of the
    // row's 4 BW holds it), else from two wavefronts' partials; then the four quarters of the chunk
    // in order, ((Q0 + Q1) + Q2) + Q3.
#pragma unroll
    for (int it = 0; it < NI; ++it)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float t = acc[it][m];
            t += dpp<kDppQuadXor1>(t);
            t += dpp<kDppQuadXor2>(t);
            t += dpp<kDppRowRor4>(t);
            if constexpr (BW == 4) t += dpp<kDppRowRor8>(t);
            if ((lane & (4 * BW - 1)) == 4 * BW - 1) red[wave][(it * kGroupRows + rr) * M + m] = t;
        }
    __syncthreads();
    if (tid < kRows * M) {
        const uint32_t r = tid / M, m = tid % M, n = row0 + r;
        auto quarter = [&](uint32_t q) {  // blocks 4q .. 4q + 3 of the chunk
            if constexpr (BW == 4) return red[q][tid];
            else return red[2 * q][tid] + red[2 * q + 1][tid];
        };
        const float v = ((quarter(0) + quarter(1)) + quarter(2)) + quarter(3);
        if (n < N) y[static_cast<uint64_t>(m) * N + n] = v;
    }
}

// ---------------------------------------------------------------------------
// Matrix-core GEMV for 3 <= M <= 8, accurate to fp32 level.
//
// Per 256-weight block the product is split as
//   sum_k x[m,k] w[n,k] = d * sum_k x[m,k] sc(k) q(k) - dmin * sum_s mn(s) sum_{k in s} x[m,k],
// and both sums run on the matrix cores in f16 with fp32 accumulation:
//  - B holds the integers sc * q (<= 45) and mn (<= 15) as the raw bits of f16
//    subnormals, i.e. v * 2^-24 exactly: 2-bit codes become f16 operands with a
//    byte permute, a mask and a 24-bit multiply, no conversion instruction;
//  - A holds x in two f16 pieces (x' = h1 + h2 to 2^-22 of |x'|), after scaling
//    each row of each block by a power of two 2^s so its largest |x| lies in
//    [2^13, 2^14). Products h * v * 2^-24 are exact in fp32.
// Codes at 2-bit position p are masked in place (value 4^p q for p < 3, 4q for
// p = 3 after a 4-bit shift), so the A pieces of position p carry the inverse
// factor 1, 1/4, 1/16 or 1/4 (exact powers of two). Each wavefront builds the A
// fragments of its own block and keeps them in registers for all its tiles.
//
// MFMA v_mfma_f32_16x16x32_f16: lane l holds A row l % 16 (m = row % 8, piece =
// row / 8) and k = 8 (l / 16) .. +7, B column l % 16 and the same k, and D
// rows 4 (l / 16) .. +3 of column l % 16. MFMA j (0..7) of a block covers code
// segment G = l / 16 (the 16 code bytes 16 G .. 16 G + 15), 2-bit position
// p = j / 2 and bytes 8 (j % 2) .. +7 of the segment: block elements
// 128 (G / 2) + 32 p + 16 (G % 2) + 8 (j % 2) + i, i < 8, all of sub-block
// 8 (G / 2) + 2 p + G % 2. The min term is one v_mfma_f32_16x16x16_f16 per
// block with k = sub-block (lane l: sub-blocks 4 (l / 16) .. +3).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kMvTiles = 4;             // 16-column tiles per workgroup
constexpr uint32_t kMvWaves = 16;

// The two f16 pieces of v0 c and v1 c (c a power of two), packed low, high:
// h1 = f16(v c) and h2 = f16(v c - h1), each one rounding of a value that is
// exact in f32 (v c scales by a power of two; v c - h1 keeps the bits h1 left),
// so they equal rounding v c to f32 and then to f16. One v_fma_mix per piece.
__device__ __forceinline__ void split_f16_pair(float v0, float v1, float c, uint32_t *b1, uint32_t *b2) {
    uint32_t h, r;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0" : "=v"(h) : "v"(v0), "v"(c));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0" : "+v"(h) : "v"(v1), "v"(c));
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,0,1]" : "=v"(r) : "v"(v0), "v"(c), "v"(h));
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "+v"(r) : "v"(v1), "v"(c), "v"(h));
    *b1 = h;
    *b2 = r;
}

// The same for one value: h1 in the low half of *b1, h2 in the low half of *b2.
__device__ __forceinline__ void split_f16_one(float v, float c, uint32_t *b1, uint32_t *b2) {
    uint32_t h, r;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0" : "=v"(h) : "v"(v), "v"(c));
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,0,1]" : "=v"(r) : "v"(v), "v"(c), "v"(h));
    *b1 = h;
    *b2 = r;
}

// Activation rows of one block in LDS: 8 rows of 256 floats per wavefront,
// rows 260 floats apart so that lanes reading different rows at the same
// column start in different banks.
constexpr uint32_t kMvXRow = 260;
constexpr uint32_t kMvXWave = 8 * kMvXRow;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A operands of one block, for lane l = 16 G + col (row m = col % 8, piece 1
// if col < 8 else 2): the eight 16x16x32 fragments, the min-term fragment and
// the inverse scales of the lane's four D rows.
struct MvA {
    f16x8 af[8];
    f16x4 am;
    f32x4 isc;
};

// Builds MvA from the lane's 32 activations xq[p][jj] = elements 8 jj + 4 half
// .. +3 of sub-block 8 (G / 2) + 2 p + G % 2 of row m (half = col / 8; lanes
// col and col ^ 8 hold the two halves of the same sixteen elements).
//  - Row maximum of |x| over the block (the eight lanes of row m), giving the
//    scale 2^s that puts it in [2^13, 2^14). A subnormal maximum counts as
//    2^-127; zero, inf or NaN maxima leave the row unscaled.
//  - Sub-block sums S, pairwise in element order: ((e0 + e1) + (e2 + e3)) for
//    each quad, then (q0 + q1) + (q2 + q3); quads 0 and 2 are lane half 0's,
//    1 and 3 half 1's, and both lanes form the same sum.
//  - Fragments: MFMA j takes elements 8 (j % 2) .. +7 of sub-block p = j / 2,
//    scaled by 2^s times the position factor (one exact power of two). Each
//    lane splits its four elements into h1 = f16(v) and h2 = f16(v - h1) (the
//    difference is exact before its one rounding), keeps the piece of its row
//    and takes the other four elements' piece from its partner by DPP.
__device__ __forceinline__ MvA mv_build_a(const f32x4 (&xq)[4][2], uint32_t G, uint32_t m, bool second) {
    MvA a;
    float mx = 0.0f, S[4];
#pragma unroll
    for (uint32_t p = 0; p < 4; ++p) {
        float q[2];
#pragma unroll
        for (uint32_t jj = 0; jj < 2; ++jj) {
            const f32x4 v = xq[p][jj];
#pragma unroll
            for (uint32_t i = 0; i < 4; ++i)
                mx = p == 0 && jj == 0 && i == 0 ? __builtin_fabsf(v[0]) : __builtin_fmaxf(mx, __builtin_fabsf(v[i]));
            q[jj] = (v[0] + v[1]) + (v[2] + v[3]);
        }
        S[p] = (q[0] + dpp<kDppRowRor8>(q[0])) + (q[1] + dpp<kDppRowRor8>(q[1]));
    }
    mx = __builtin_fmaxf(mx, dpp<kDppRowRor8>(mx));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
    int sx = 0;
    if (mx > 0.0f && mx <= 3.4e38f) {
        const int e = static_cast<int>(__builtin_bit_cast(uint32_t, mx) >> 23) - 127;
        sx = 13 - e;
        sx = sx < -100 ? -100 : (sx > 100 ? 100 : sx);
    }
    const float fwd = __builtin_bit_cast(float, static_cast<uint32_t>(127 + sx) << 23);
    const float inv = __builtin_bit_cast(float, static_cast<uint32_t>(127 - sx) << 23);
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) {
        const uint32_t p = j >> 1;
        // The product differs from scaling twice only below f32's normal range, where both pieces are
        // zero in f16 anyway.
        const float c = fwd * (p == 0 ? 1.0f : (p == 2 ? 0.0625f : 0.25f));
        const f32x4 v = xq[p][j & 1u];
        u32x4 frag;
#pragma unroll
        for (uint32_t i = 0; i < 2; ++i) {
            uint32_t b1, b2;
            split_f16_pair(v[2 * i], v[2 * i + 1], c, &b1, &b2);
            // Elements 2i, 2i + 1 of the eight are lane half 0's: piece 1 lanes (DPP banks 0, 1) keep h1,
            // piece 2 lanes (banks 2, 3) take the partner's h2. Elements 4 + 2i, 5 + 2i the other way round.
            frag[i] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(b1), static_cast<int>(b2),
                                                                        kDppRowRor8, 0xF, 0xC, false));
            frag[2 + i] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(b2), static_cast<int>(b1),
                                                                            kDppRowRor8, 0xF, 0x3, false));
        }
        a.af[j] = __builtin_bit_cast(f16x8, frag);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Min-term fragment: sub-blocks 4 G .. 4 G + 3 of row m. Sub-block 4 G + i is S[2 (G % 2) + i / 2] of
    // the lanes of segment 2 (G / 2) + i % 2, and a lane of half h offers S[2 h + q] as its q-th sum.
    const float s01[2] = {second ? S[2] : S[0], second ? S[3] : S[1]};
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const int src = static_cast<int>(16u * (2u * (G >> 1) + (i & 1u)) + m + 8u * (G & 1u));
        const float sub = __shfl(s01[i >> 1], src, 64);
        uint32_t h1, h2;  // |sum| < 2^18: scaled by 2^-5 into f16 range
        split_f16_one(sub, fwd * 0.03125f, &h1, &h2);
        a.am[i] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(second ? h2 : h1));
    }
    // Inverse scales of D rows 4 (G % 2) .. +3 (activation rows of lanes 0..7).
#pragma unroll
    for (uint32_t v = 0; v < 4; ++v) a.isc[v] = __shfl(inv, static_cast<int>(4u * (G & 1u) + v), 64);
    return a;
}

// One block of one 16-column tile: the lane's 16 code bytes qv (segment G of
// column col), its half's scale bytes scv (8 (G / 2) ..), the min nibbles of
// sub-blocks 4 G .. +3 (mnv) and d, dmin (ddv); adds the block's products,
// scaled back, to acc (D rows 4 G .. +3 of column col).
__device__ __forceinline__ void mv_tile(const MvA &a, u32x4 qv, u32x2 scv, uint32_t mnv, uint32_t ddv, uint32_t G,
                                        f32x4 &acc) {
    uint32_t u[8];
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        u[2 * i] = __builtin_amdgcn_perm(0u, qv[i], 0x0c010c00u);      // bytes 0, 1 -> 16-bit slots
        u[2 * i + 1] = __builtin_amdgcn_perm(0u, qv[i], 0x0c030c02u);  // bytes 2, 3
    }
    const uint32_t sh = 8u * (G & 1u);
    const uint32_t sc[4] = {(scv[0] >> sh) & 15u, (scv[0] >> (sh + 16u)) & 15u, (scv[1] >> sh) & 15u,
                            (scv[1] >> (sh + 16u)) & 15u};
    f32x4 d1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) {
        const uint32_t p = j >> 1, jj = j & 1u;
        const uint32_t mask = p == 0 ? 0x00030003u : (p == 2 ? 0x00300030u : 0x000C000Cu);
        u32x4 bv;
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i) {
            const uint32_t vv = p == 3 ? u[4 * jj + i] >> 4 : u[4 * jj + i];
            bv[i] = __umul24(vv & mask, sc[p]);
        }
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.af[j], __builtin_bit_cast(f16x8, bv), d1, 0, 0, 0);
    }
    u32x2 bm;
    bm[0] = (__builtin_amdgcn_perm(0u, mnv, 0x0c010c00u) >> 4) & 0x000F000Fu;
    bm[1] = (__builtin_amdgcn_perm(0u, mnv, 0x0c030c02u) >> 4) & 0x000F000Fu;
    const f32x4 d2 = __builtin_amdgcn_mfma_f32_16x16x16f16(a.am, __builtin_bit_cast(f16x4, bm),
                                                          f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    const float dl = f16_low(ddv) * 16777216.0f;    // d * 2^24
    const float ml = f16_high(ddv) * 536870912.0f;  // dmin * 2^24 * 2^5
#pragma unroll
    for (uint32_t v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(a.isc[v], __builtin_fmaf(-ml, d2[v], dl * d1[v]), acc[v]);
}

// The workgroup's partial sums: lane l of wavefront w holds D rows 4 G + v
// (piece G / 2 of activation row m = 4 (G % 2) + v) of column l % 16 of each
// tile; they meet in LDS (part, at w * stride) and are added in wavefront
// order, piece 1 before piece 2. The caller has made part free.
__device__ __forceinline__ void mv_store(const f32x4 (&acc)[kMvTiles], float *part, uint32_t stride, uint32_t tid,
                                         uint32_t wave, uint32_t G, uint32_t col, float *y, uint32_t M, uint32_t N,
                                         uint32_t row0) {
#pragma unroll
    for (uint32_t t = 0; t < kMvTiles; ++t)
#pragma unroll
        for (uint32_t v = 0; v < 4; ++v) part[wave * stride + t * 256u + (4u * G + v) * 16u + col] = acc[t][v];
    __syncthreads();
    if (tid < kMvTiles * 128u) {
        const uint32_t t = tid >> 7, q = tid & 127u, mm = q >> 4, c = q & 15u, n = row0 + 16u * t + c;
        const float *rs = part + t * 256u;
        float s = rs[q] + rs[q + 128u];
#pragma unroll
        for (uint32_t wv = 1; wv < kMvWaves; ++wv) s += rs[wv * stride + q] + rs[wv * stride + q + 128u];
        if (mm < M && n < N) y[static_cast<uint64_t>(mm) * N + n] = s;
    }
}

// The lane's 32 activations (see mv_build_a) from a wavefront's LDS copy of
// the block's 8 rows.
__device__ __forceinline__ void mv_read_x(const float *xw, uint32_t G, uint32_t m, uint32_t half, f32x4 (&xq)[4][2]) {
#pragma unroll
    for (uint32_t p = 0; p < 4; ++p)
#pragma unroll
        for (uint32_t jj = 0; jj < 2; ++jj)
            xq[p][jj] = *reinterpret_cast<const f32x4 *>(xw + m * kMvXRow + 128u * (G >> 1) + 16u * (G & 1u) + 32u * p +
                                                         8u * jj + 4u * half);
}

// K < 4096 (nb = K / 256 < 16 blocks): wavefront w < nb * (16 / nb) takes
// block w % nb of the tiles t with t % (16 / nb) == w / nb (set by the host as
// wpb = 16 / nb, active = nb * wpb).
struct MvPlan {
    uint32_t wpb, active;
};

// grid (ceil(N / (16 kMvTiles)), problems); 1024 threads = 16 wavefronts.
// Each active wavefront copies its block's 8 activation rows into its own LDS
// region (direct buffer-to-LDS loads, issued before its weight loads so they
// land first), loads its tiles' weight bytes straight into registers and
// builds the block's A fragments from the LDS copy.
__global__ __launch_bounds__(1024) void k_gemv_mfma(const float *__restrict__ x, const uint8_t *__restrict__ w,
                                                   float *__restrict__ y, uint32_t M, uint32_t N, uint32_t K,
                                                   GemvBatch bt, MvPlan plan) {
    __shared__ __attribute__((aligned(16))) float lds[kMvWaves * kMvXWave];
    static_assert(kMvXWave >= kMvTiles * 256, "the partial sums reuse the activation rows");
    x += blockIdx.y * bt.x_elems;
    w += blockIdx.y * bt.w_bytes;
    y += blockIdx.y * bt.y_elems;
    const uint32_t nb = K >> 8, row_bytes = nb * kBlockBytes;
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t col = lane & 15u, G = lane >> 4;
    const uint32_t row0 = blockIdx.x * (16u * kMvTiles);
    const uint32_t nrows = min(16u * kMvTiles, N - row0);
    // Rows past N (weights) or M (activations) lie beyond these descriptors and read as zeros.
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(w + static_cast<uint64_t>(row0) * row_bytes, nrows * row_bytes);
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, M * K * 4u);
    float *const xw = lds + wave * kMvXWave;
    const uint32_t m = col & 7u;
    const bool second = col >= 8u;

    f32x4 acc[kMvTiles];
#pragma unroll
    for (uint32_t t = 0; t < kMvTiles; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const uint32_t tl = wave / nb, b = wave % nb;
    if (wave < plan.active) {
#pragma unroll
        for (uint32_t r = 0; r < 8; ++r) {
            const uint32_t u = __builtin_amdgcn_readfirstlane((r * K + 256u * b) * 4u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void *)(xw + r * kMvXRow),
                                                     16, static_cast<int>(u + 16u * lane), 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        u32x4 qv[kMvTiles];
        u32x2 scv[kMvTiles];
        uint32_t mnv[kMvTiles], ddv[kMvTiles];
#pragma unroll
        for (uint32_t t = 0; t < kMvTiles; ++t) {
            if (t % plan.wpb != tl) continue;
            const uint32_t off = (16u * t + col) * row_bytes + b * kBlockBytes;
            qv[t] = __builtin_amdgcn_raw_buffer_load_b128(wr, off + 16u + 16u * G, 0, 0);
            scv[t] = __builtin_amdgcn_raw_buffer_load_b64(wr, off + 8u * (G >> 1), 0, 0);
            mnv[t] = __builtin_amdgcn_raw_buffer_load_b32(wr, off + 4u * G, 0, 0);
            ddv[t] = __builtin_amdgcn_raw_buffer_load_b32(wr, off + 80u, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // The weight loads depend on the plan, so wait for all of them.
        vm_wait<0>();
        __builtin_amdgcn_sched_barrier(0);
        f32x4 xq[4][2];
        mv_read_x(xw, G, m, second ? 1u : 0u, xq);
        const MvA a = mv_build_a(xq, G, m, second);
#pragma unroll
        for (uint32_t t = 0; t < kMvTiles; ++t) {
            if (t % plan.wpb != tl) continue;
            mv_tile(a, qv[t], scv[t], mnv[t], ddv[t], G, acc[t]);
        }
    }
    // The partial sums reuse the activation rows once every wavefront is done with them.
    __syncthreads();
    mv_store(acc, lds, kMvXWave, tid, wave, G, col, y, M, N, row0);
}

// K = 4096 (16 blocks): the weights go through LDS. Wavefront w takes block
// w, and the workgroup copies its 64 rows (1344 contiguous bytes each) into
// LDS with dword buffer-to-LDS loads, each reading 256 contiguous bytes of one
// row: far fewer cache lines than per-lane loads of codes, scales, mins and d,
// which touch every row's lines four times. The LDS holds each wavefront's 8
// activation rows (copied 1 KiB per instruction) and tile 0's rows; once a
// wavefront has its activations in registers, its region takes its rows of
// tiles 1..3, whose bytes arrive while the A fragments are built. Wavefront w
// copies row 16 t + w of every tile t; a barrier per tile makes its rows
// visible (a plain s_barrier after a counted wait: __syncthreads would wait
// for every copy still in flight).
//
// LDS row stride in dwords: 336 (16 blocks of 21 dwords) plus 3, odd, so a
// wavefront's operand reads (16 rows x 4 segments) fall at most two to a
// bank. Rows of tiles 1..3 sit in wavefront w's activation region at
// 339 (t - 1) + 35 w: with the region stride 2080 = 32 (mod 64) the rows of
// consecutive columns land 3 banks apart.
constexpr uint32_t kMvStageRow = 339;
constexpr uint32_t kMvStageSkew = 35;
static_assert(2u * kMvStageRow + 336u + kMvStageSkew * 15u <= kMvXWave, "three staged rows fit an activation region");

__global__ __launch_bounds__(1024) void k_gemv_mfma_staged(const float *__restrict__ x, const uint8_t *__restrict__ w,
                                                          float *__restrict__ y, uint32_t M, uint32_t N, GemvBatch bt) {
    constexpr uint32_t K = 4096, row_bytes = 16u * kBlockBytes;
    __shared__ __attribute__((aligned(16))) uint32_t stage[kMvWaves * kMvXWave + 16u * kMvStageRow];
    static_assert(kMvXWave >= kMvTiles * 256, "the partial sums reuse the activation rows");
    x += blockIdx.y * bt.x_elems;
    w += blockIdx.y * bt.w_bytes;
    y += blockIdx.y * bt.y_elems;
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t col = lane & 15u, G = lane >> 4;
    const uint32_t row0 = blockIdx.x * (16u * kMvTiles);
    const uint32_t nrows = min(16u * kMvTiles, N - row0);
    // Rows past N (weights) or M (activations) lie beyond these descriptors and read as zeros.
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(w + static_cast<uint64_t>(row0) * row_bytes, nrows * row_bytes);
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, M * K * 4u);
    float *const xw = reinterpret_cast<float *>(stage) + wave * kMvXWave;
    uint32_t *const tile0 = stage + kMvWaves * kMvXWave;
    const uint32_t m = col & 7u, b = wave;
    const bool second = col >= 8u;

    // Activation rows 0..7 of block b (1 KiB each, 16 bytes a lane), then row `wave` of tile 0 (336 dwords in
    // six dword loads, the last covering 16).
#pragma unroll
    for (uint32_t r = 0; r < 8; ++r) {
        const uint32_t u = __builtin_amdgcn_readfirstlane((r * K + 256u * b) * 4u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void *)(xw + r * kMvXRow), 16,
                                                 static_cast<int>(u + 16u * lane), 0, 0, 0);
    }
#pragma unroll
    for (uint32_t k = 0; k < 6; ++k)
        if (k < 5u || lane < 16u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (__attribute__((address_space(3))) void *)(tile0 + wave * kMvStageRow + 64u * k), 4,
                static_cast<int>(wave * row_bytes + 4u * (64u * k + lane)), 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // Loads complete in issue order: the activations are in once at most tile 0's six copies are in flight.
    vm_wait<6>();
    __builtin_amdgcn_sched_barrier(0);
    f32x4 xq[4][2];
    mv_read_x(xw, G, m, second ? 1u : 0u, xq);
    // The region is free once these reads are done: row `wave` of tiles 1..3 goes there.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (uint32_t t = 1; t < kMvTiles; ++t) {
        const uint32_t r = 16u * t + wave;
#pragma unroll
        for (uint32_t k = 0; k < 6; ++k)
            if (k < 5u || lane < 16u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr,
                    (__attribute__((address_space(3))) void *)(reinterpret_cast<uint32_t *>(xw) + (t - 1u) * kMvStageRow +
                                                               kMvStageSkew * wave + 64u * k),
                    4, static_cast<int>(r * row_bytes + 4u * (64u * k + lane)), 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    const MvA a = mv_build_a(xq, G, m, second);
    f32x4 acc[kMvTiles];
#pragma unroll
    for (uint32_t t = 0; t < kMvTiles; ++t) {
        // Tile t's rows are in LDS once this wavefront's copies of them are done (they complete in issue
        // order: six per tile) and every wavefront has passed the barrier.
        __builtin_amdgcn_sched_barrier(0);
        vm_wait_n<6 * (kMvTiles - 1)>(6u * (kMvTiles - 1u - t));
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t *blk =
            (t == 0 ? tile0 + col * kMvStageRow : stage + col * kMvXWave + (t - 1u) * kMvStageRow + kMvStageSkew * col) +
            wave * (kBlockBytes / 4u);
        const u32x4 qv = {blk[4u + 4u * G], blk[5u + 4u * G], blk[6u + 4u * G], blk[7u + 4u * G]};
        const u32x2 scv = {blk[2u * (G >> 1)], blk[2u * (G >> 1) + 1u]};
        acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        mv_tile(a, qv, scv, blk[G], blk[20], G, acc[t]);
    }
    // Every wavefront is done with the LDS before the partial sums reuse it.
    __syncthreads();
    mv_store(acc, reinterpret_cast<float *>(stage), kMvTiles * 256u, tid, wave, G, col, y, M, N, row0);
}

// K > 4096 (more than 16 blocks): wavefront w takes blocks w, w + 16, ... and
// copies exactly the bytes it decodes, its block of the workgroup's 64 rows
// (84 contiguous bytes each), with dword buffer-to-LDS loads: six per 16-row
// tile, each reading about three rows' blocks. No wavefront reads another's
// LDS, so there is no barrier: tile t's arithmetic starts as soon as the
// wavefront's own copies of it have landed (they complete in issue order),
// and wavefronts never wait for each other between blocks. The activations
// are copied as in k_gemv_mfma_staged; tile 0 has a slot of its own per
// wavefront, tiles 1..3 take the wavefront's activation region once the
// activations are in registers. A tile's 16 rows are 21 dwords apart (the
// block itself): an odd stride, so operand reads fall at most two to a bank.
// With several blocks per wavefront this beats the row copies and their
// per-tile barriers (M=8, N=4096, K=14336: 26.4 us against 32.1 us), while for
// K = 4096 the row copies touch fewer cache lines (11.1 us against 11.4 us at
// N=14336).
constexpr uint32_t kMvOwnTile = 16u * (kBlockBytes / 4u);  // 336 dwords: one block of 16 rows
static_assert(3u * kMvOwnTile <= kMvXWave, "tiles 1..3 fit an activation region");

__global__ __launch_bounds__(1024) void k_gemv_mfma_blocks(const float *__restrict__ x, const uint8_t *__restrict__ w,
                                                          float *__restrict__ y, uint32_t M, uint32_t N, uint32_t K,
                                                          GemvBatch bt) {
    __shared__ __attribute__((aligned(16))) uint32_t stage[kMvWaves * (kMvXWave + kMvOwnTile)];
    static_assert(kMvXWave >= kMvTiles * 256, "the partial sums reuse the activation rows");
    x += blockIdx.y * bt.x_elems;
    w += blockIdx.y * bt.w_bytes;
    y += blockIdx.y * bt.y_elems;
    const uint32_t nb = K >> 8, row_bytes = nb * kBlockBytes;
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t col = lane & 15u, G = lane >> 4;
    const uint32_t row0 = blockIdx.x * (16u * kMvTiles);
    const uint32_t nrows = min(16u * kMvTiles, N - row0);
    // Rows past N (weights) or M (activations) lie beyond these descriptors and read as zeros.
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(w + static_cast<uint64_t>(row0) * row_bytes, nrows * row_bytes);
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, M * K * 4u);
    float *const xw = reinterpret_cast<float *>(stage) + wave * kMvXWave;
    uint32_t *const own0 = stage + kMvWaves * kMvXWave + wave * kMvOwnTile;
    const uint32_t m = col & 7u;
    const bool second = col >= 8u;
    // Dword d of a tile copy is word d % 21 of row d / 21's block.
    uint32_t coff[6];
#pragma unroll
    for (uint32_t k = 0; k < 6; ++k) {
        const uint32_t d = 64u * k + lane;
        coff[k] = (d / 21u) * row_bytes + 4u * (d % 21u);
    }

    f32x4 acc[kMvTiles];
#pragma unroll
    for (uint32_t t = 0; t < kMvTiles; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (uint32_t b = wave; b < nb; b += kMvWaves) {
        // The previous block's LDS reads are done before its regions are overwritten.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (uint32_t r = 0; r < 8; ++r) {
            const uint32_t u = __builtin_amdgcn_readfirstlane((r * K + 256u * b) * 4u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void *)(xw + r * kMvXRow), 16,
                                                     static_cast<int>(u + 16u * lane), 0, 0, 0);
        }
#pragma unroll
        for (uint32_t k = 0; k < 6; ++k)
            if (k < 5u || lane < 16u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void *)(own0 + 64u * k), 4,
                                                         static_cast<int>(b * kBlockBytes + coff[k]), 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        vm_wait<6>();
        __builtin_amdgcn_sched_barrier(0);
        f32x4 xq[4][2];
        mv_read_x(xw, G, m, second ? 1u : 0u, xq);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t t = 1; t < kMvTiles; ++t)
#pragma unroll
            for (uint32_t k = 0; k < 6; ++k)
                if (k < 5u || lane < 16u)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        wr,
                        (__attribute__((address_space(3))) void *)(reinterpret_cast<uint32_t *>(xw) + (t - 1u) * kMvOwnTile +
                                                                   64u * k),
                        4, static_cast<int>(16u * t * row_bytes + b * kBlockBytes + coff[k]), 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        const MvA a = mv_build_a(xq, G, m, second);
#pragma unroll
        for (uint32_t t = 0; t < kMvTiles; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            vm_wait_n<6 * (kMvTiles - 1)>(6u * (kMvTiles - 1u - t));
            asm volatile("" ::: "memory");  // the LDS reads below stay after the wait
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t *blk = (t == 0 ? own0 : reinterpret_cast<const uint32_t *>(xw) + (t - 1u) * kMvOwnTile) +
                                  col * (kBlockBytes / 4u);
            const u32x4 qv = {blk[4u + 4u * G], blk[5u + 4u * G], blk[6u + 4u * G], blk[7u + 4u * G]};
            const u32x2 scv = {blk[2u * (G >> 1)], blk[2u * (G >> 1) + 1u]};
            mv_tile(a, qv, scv, blk[G], blk[20], G, acc[t]);
        }
    }
    // Every wavefront is done with the LDS before the partial sums reuse it.
    __syncthreads();
    mv_store(acc, reinterpret_cast<float *>(stage), kMvTiles * 256u, tid, wave, G, col, y, M, N, row0);
}

// ---------------------------------------------------------------------------
// Matrix-core path for M > 8: y = bf16(x) * bf16(W)^T with fp32 accumulation.
//
// k_x_to_bf16 rounds the activations to bf16 (nearest even) once, into a
// workspace. k_gemm_q2k then computes a 128 (M) x 256 (N) tile of y per
// 512-thread workgroup: two groups of four wavefronts split K in halves, and
// wavefront w of a group owns columns 64w .. 64w+63 of the tile for all 128
// rows, as a 4 x 2 grid of v_mfma_f32_32x32x16_bf16 accumulators. K advances
// 64 weights per step (a quarter super-block). Activation tiles (128 x 64
// bf16) and each wavefront's raw weight blocks reach LDS through direct
// buffer-to-LDS loads; each wavefront decodes its own 64 columns from LDS into
// MFMA B fragments one slice ahead of the MFMAs that use them, so the decode
// arithmetic overlaps the matrix cores. One workgroup barrier per step.
//
// Inside a step the 64 k are taken in an order that suits the code bytes: the
// k-chunk of 8 that MFMA slice kk gives to lane half kh (lanes 32kh .. 32kh+31)
// is chunk 4 (kk / 2) + 2 kh + kk % 2 of the step, i.e. 2-bit position
// 2 (j % 2) + kk / 2 (j = quarter of the block), code segment kh, code bytes
// 8 (kk % 2) .. +7 of that segment. Activations are read from LDS in the same
// order, so every product pairs x[m, k] with w[n, k].
constexpr uint32_t kGM = 128, kGN = 256;

__device__ __forceinline__ bf16x8 pack_bf16(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                            float a7) {
    bf16x8 v;
    v[0] = static_cast<__bf16>(a0);
    v[1] = static_cast<__bf16>(a1);
    v[2] = static_cast<__bf16>(a2);
    v[3] = static_cast<__bf16>(a3);
    v[4] = static_cast<__bf16>(a4);
    v[5] = static_cast<__bf16>(a5);
    v[6] = static_cast<__bf16>(a6);
    v[7] = static_cast<__bf16>(a7);
    return v;
}

// Each thread converts kXU chunks of 8 values per round, all loads first, so a
// few hundred workgroups keep the whole 8 MB in flight (launching thousands of
// small workgroups costs more than the copy itself at this size).
constexpr uint32_t kXU = 4;

__global__ __launch_bounds__(256) void k_x_to_bf16(const float4 *__restrict__ x, bf16x8 *__restrict__ xb,
                                                   uint64_t n8) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    const uint64_t t = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint64_t base = 0;
    // Whole rounds: every thread's kXU chunks are in range.
    for (; base + kXU * stride <= n8; base += kXU * stride) {
        float4 a[kXU], b[kXU];
#pragma unroll
        for (uint32_t u = 0; u < kXU; ++u) {
            const uint64_t i = base + u * stride + t;
            a[u] = x[2 * i];
            b[u] = x[2 * i + 1];
        }
#pragma unroll
        for (uint32_t u = 0; u < kXU; ++u)
            xb[base + u * stride + t] = pack_bf16(a[u].x, a[u].y, a[u].z, a[u].w, b[u].x, b[u].y, b[u].z, b[u].w);
    }
    for (uint64_t i = base + t; i < n8; i += stride) {
        const float4 a = x[2 * i], b = x[2 * i + 1];
        xb[i] = pack_bf16(a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w);
    }
}

// Workgroups are dealt to the eight XCDs in turn (XCD = id % 8). When the tile
// count allows, each XCD gets a contiguous band of N tiles with all their M
// tiles, so the W rows its workgroups share stay in that XCD's L2.
__device__ __forceinline__ void gemm_tile(uint32_t b, uint32_t tiles_m, uint32_t tiles_n, uint32_t *tm,
                                          uint32_t *tn) {
    const uint32_t total = tiles_m * tiles_n;
    uint32_t idx = b;
    if (total % 8 == 0) idx = (b / 8) + (b % 8) * (total / 8);
    *tn = idx / tiles_m;
    *tm = idx % tiles_m;
}

// Raw bytes of one half super-block for one lane: for each of its two columns
// the lane's 16-byte code segment and the half's 8 scale bytes, plus d, dmin.
struct GemmRaw {
    uint32_t q[2][4];
    uint32_t sc[2][2];
    uint32_t dd[2];
};

// Expert-routed mode: tile tm of the M dimension is tiles[tm], a run of
// rows of the expert-ordered activations (bf16, p0 .. p0 + count - 1) that
// all use one expert's weights; row p of the run is written to output row
// perm[p]. Unused tile entries (count 0) end their workgroups at once.
struct GemmRoute {
    const MoeTile *tiles;
    const uint32_t *perm;
    uint64_t expert_stride;
};
static_assert(kGM == kMoeTileRows, "routing tiles must match the GEMM's M tile");

// Wait until at most N vector-memory operations of this wavefront are still in
// flight, then meet the rest of the workgroup (gfx9 s_waitcnt: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their "no wait" maxima). The
// barrier is a compiler memory barrier too, so no LDS access moves across it.
template <uint32_t N>
__device__ __forceinline__ void vm_barrier() {
    static_assert(N < 64, "vmcnt has six bits");
    __builtin_amdgcn_s_waitcnt(static_cast<int>((N & 15u) | ((N >> 4) << 14) | 0x0F70u));
    asm volatile("s_barrier" ::: "memory");
}

// Weight staging in LDS (per group and block): wavefront wq's 64 columns fill
// 22 runs of 65 dwords. Run j holds columns 3 j, 3 j + 1, 3 j + 2 of the
// wavefront as 21 dwords each (the whole 84-byte block) and one pad dword;
// run 21 holds only column 63 (its other slots are filled and never read).
// The 65-dword run stride spreads the columns a fragment reads over the banks.
constexpr uint32_t kWRun = 65, kWRuns = 22;
constexpr uint32_t kWWave = kWRun * kWRuns;  // dwords per wavefront and block
constexpr uint32_t kWGroup = 4 * kWWave;     // dwords per group and block

template <bool kRouted>
__global__ __launch_bounds__(512) void k_gemm_q2k(const __bf16 *__restrict__ xb, const uint8_t *__restrict__ w,
                                                  float *__restrict__ y, uint32_t M, uint32_t N, uint32_t K,
                                                  uint32_t tiles_m, GemmRoute rg) {
    // Eight wavefronts, two per SIMD: group g = wave / 4 runs the MFMAs of K
    // half g (blocks g nblk .. g nblk + nblk - 1) for the whole 128 x 256 tile;
    // wavefront wave % 4 owns columns 64 (wave % 4) .. +63.
    //
    // Both operands reach LDS by direct buffer-to-LDS loads (the LDS bit of a
    // buffer load: no registers on the way). Activations: two stage buffers
    // per group of 128 rows x 64 bf16 (16 KiB), one 64-k step ahead. Weights:
    // two block buffers per group, whole 84-byte blocks copied as contiguous
    // dwords, one block ahead. Copying whole blocks keeps each load
    // instruction on a few cache lines; a wavefront fetching its fragments'
    // bytes straight from memory touches 32 rows per instruction, and the
    // per-line cost of that dominated the kernel. At the end the same memory
    // carries the partial sums the groups exchange.
    constexpr uint32_t kStepK = 64;
    constexpr uint32_t kTile = kGM * kStepK;  // bf16 per group and stage
    __shared__ __attribute__((aligned(16))) __bf16 xs0[2 * kTile], xs1[2 * kTile];
    __shared__ __attribute__((aligned(16))) uint32_t ws0[2 * kWGroup], ws1[2 * kWGroup];
    static_assert(2 * kTile * 2 == 2 * 64 * 64 * 4 && 2 * kWGroup * 4 >= 2 * 64 * 64 * 4,
                  "the partial-sum exchange needs 16 KiB per wavefront");

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t grp = wave >> 2, wq = wave & 3u;
    const uint32_t kh = lane >> 5, col = lane & 31u;
    uint32_t tm, tn;
    if constexpr (kRouted) {
        // Routing tiles in list order (full tiles first, partial ones last), all N
        // tiles of one routing tile in turn: the short tiles run at the end and
        // fill the last round of workgroups. With a multiple of 8 N tiles, N tile
        // tn always lands on XCD tn % 8, so an expert's weight rows stay in one
        // XCD's L2.
        const uint32_t tiles_n = (N + kGN - 1) / kGN;
        tm = blockIdx.x / tiles_n;
        tn = blockIdx.x % tiles_n;
    } else {
        gemm_tile(blockIdx.x, tiles_m, (N + kGN - 1) / kGN, &tm, &tn);
    }
    const uint32_t n0 = tn * kGN;
    const uint32_t nb = K >> 8, row_bytes = nb * kBlockBytes;
    // rows: valid rows of the tile; xt, wt: its activations and weight matrix.
    __shared__ uint32_t rowmap[kGM];
    uint32_t m0 = 0, rows;
    const __bf16 *xt;
    const uint8_t *wt;
    if constexpr (kRouted) {
        const MoeTile t = rg.tiles[tm];
        if (t.count == 0) return;
        rows = t.count;
        xt = xb + static_cast<uint64_t>(t.p0) * K;
        wt = w + t.expert * rg.expert_stride;
        if (tid < kGM) rowmap[tid] = tid < rows ? rg.perm[t.p0 + tid] : 0u;
    } else {
        m0 = tm * kGM;
        rows = min(kGM, M - m0);
        xt = xb + static_cast<uint64_t>(m0) * K;
        wt = w;
    }
    // Group g takes blocks kb0 .. kb0 + nblk - 1. With an odd block count the
    // last block of group 1 does not exist; that group then only meets the
    // barriers of its last block.
    const uint32_t nblk = (nb + 1) >> 1, kb0 = grp * nblk;

    // Rows past M or N lie beyond these descriptors and load as zeros.
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(xt, rows * K * 2u);
    const __amdgpu_buffer_rsrc_t wr =
        buffer_rsrc(wt + static_cast<uint64_t>(n0) * row_bytes, min(kGN, N - n0) * row_bytes);

    // Activation loads: instruction i of wavefront wq fills the 64 16-byte
    // slots 64 (4 wq + i) + lane of the group's stage tile, i.e. tile row
    // r = 32 wq + 8 i + lane / 8, stored chunk lane % 8, which receives
    // activation chunk (lane % 8) ^ ((r / 2) % 8) of the step (8 bf16). Rows
    // are 128 B with no padding. A fragment read serves 16 lanes (16
    // consecutive rows, one chunk each) per pass over the 64 banks; the XOR
    // key (r / 2) % 8 gives the 8 even and the 8 odd rows 8 different chunk
    // slots, so the 16 reads hit 16 different 4-bank groups. The whole offset
    // goes in the lane offset, which the descriptor's range check covers.
    const uint32_t xrow = (32u * wq + (lane >> 3)) * K * 2u;
    const uint32_t xv0 = xrow + 16u * ((lane & 7u) ^ (lane >> 4));       // even i: key lane / 16
    const uint32_t xv1 = xrow + 16u * ((lane & 7u) ^ (4u + (lane >> 4)));  // odd i: key 4 + lane / 16
    // Step s of the group is K step 4 kb0 + s (64 k each).
    auto dma_x = [&](__bf16 *stage, uint32_t s, uint32_t i) __attribute__((always_inline)) {
        __bf16 *dst = stage + grp * kTile + 4u * wq * 512u + 512u * i;
        // The uniform part is summed in scalar registers first, so that the
        // per-instruction lane offsets are not hoisted out of the loop.
        const uint32_t u = __builtin_amdgcn_readfirstlane(i * 8u * K * 2u + (4u * kb0 + s) * 128u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void *)dst, 16,
                                                 static_cast<int>((i & 1u ? xv1 : xv0) + u), 0, 0, 0);
    };

    // Weight loads, one dword per lane: in run j, lane l takes dword l % 21
    // of column 3 j + l / 21 (lane 63 repeats lane 62's dword into the pad).
    const uint32_t wl = lane == 63u ? 62u : lane;
    const uint32_t wv = (64u * wq + wl / 21u) * row_bytes + 4u * (wl % 21u);
    auto dma_w = [&](uint32_t *buf, uint32_t kb, uint32_t j) __attribute__((always_inline)) {
        uint32_t *dst = buf + grp * kWGroup + wq * kWWave + kWRun * j;
        const uint32_t u = __builtin_amdgcn_readfirstlane(3u * j * row_bytes + kb * kBlockBytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void *)dst, 4,
                                                 static_cast<int>(wv + u), 0, 0, 0);
    };

    // This lane's two columns (32 jj + col of the wavefront) in a block buffer.
    uint32_t wcol[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const uint32_t c = 32u * jj + col;
        wcol[jj] = grp * kWGroup + wq * kWWave + kWRun * (c / 3u) + 21u * (c % 3u);
    }
    // Half-block h's bytes for both columns: the lane's 16-byte code segment,
    // the half's 8 scale bytes, d and dmin.
    auto read_raw = [&](GemmRaw &r, const uint32_t *buf, uint32_t h) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const uint32_t *c = buf + wcol[jj];
#pragma unroll
            for (int e = 0; e < 4; ++e) r.q[jj][e] = c[4u + 8u * h + 4u * kh + e];
            r.sc[jj][0] = c[2u * h];
            r.sc[jj][1] = c[2u * h + 1u];
            r.dd[jj] = c[20];
        }
    };

    // B fragments of MFMA slice kk (0..7) of a half-block, both columns: 2-bit
    // position p = kk / 2, code bytes 8 (kk % 2) .. +7 of segment kh. All 16
    // weights of a sub-block share d * sc and dmin * mn, so a weight takes one
    // of four values: w(q) = RN(d*sc*q - dmin*mn) for q = 0..3 (d*sc*q and
    // dmin*mn are exact, the fma rounds once, as the decode rule does), then
    // rounded to bf16. Those four bf16 values form an 8-byte table (w0 w1 in
    // one dword, w2 w3 in the other), built when the sub-block's first slice
    // (kk even) is decoded and kept for its second. Each code selects its
    // entry with a byte permute: masked to 2q per byte, the codes become the
    // selector bytes 2q, 2q + 1 of two table bytes. Slices are always decoded
    // in the order 0, 1, 2, ..., so the table in hand is the sub-block's.
    uint32_t lut[2][2];
    auto decode = [&](const GemmRaw &r, int kk, bf16x8 (&b)[2]) __attribute__((always_inline)) {
        const int p = kk >> 1, ih = kk & 1;
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            if (ih == 0) {
                // Scale byte 2p + kh: the low nibble scales d, the high one dmin.
                const uint32_t sh = 8u * kh + 16u * static_cast<uint32_t>(p & 1);
                const float sc = static_cast<float>(__builtin_amdgcn_ubfe(r.sc[jj][p >> 1], sh, 4));
                const float mn = static_cast<float>(__builtin_amdgcn_ubfe(r.sc[jj][p >> 1], sh + 4u, 4));
                const float dl = f16_low(r.dd[jj]) * sc, ml = f16_high(r.dd[jj]) * mn;
                // w(0) as fma(dl, 0, -ml), not -ml: an infinite or NaN dl must make it NaN, as
                // d*sc*0 - dmin*mn is in the decode rule.
                const bf16x2 w01 = {static_cast<__bf16>(__builtin_fmaf(dl, 0.0f, -ml)), static_cast<__bf16>(dl - ml)};
                const bf16x2 w23 = {static_cast<__bf16>(__builtin_fmaf(dl, 2.0f, -ml)),
                                    static_cast<__bf16>(__builtin_fmaf(dl, 3.0f, -ml))};
                lut[jj][0] = __builtin_bit_cast(uint32_t, w01);
                lut[jj][1] = __builtin_bit_cast(uint32_t, w23);
            }
            u32x4 o;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // Four weights from one code dword: bytes 2q (m2) and 2q + 1 (m3), interleaved
                // into per-weight selector pairs, pick their bf16 entries from the table.
                const uint32_t v = r.q[jj][2 * ih + t];
                const uint32_t m2 = (p == 0 ? (v << 1) : (v >> (2 * p - 1))) & 0x06060606u;
                const uint32_t m3 = m2 | 0x01010101u;
                o[2 * t] = __builtin_amdgcn_perm(lut[jj][1], lut[jj][0], __builtin_amdgcn_perm(m3, m2, 0x05010400u));
                o[2 * t + 1] = __builtin_amdgcn_perm(lut[jj][1], lut[jj][0], __builtin_amdgcn_perm(m3, m2, 0x07030602u));
            }
            b[jj] = __builtin_bit_cast(bf16x8, o);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.0f;

    // A fragment of slice kq (0..3 within a 64-k step), row block i: tile row
    // 32 i + col, activation chunk c = 4 (kq / 2) + 2 kh + kq % 2 of the step,
    // stored as chunk c ^ ((col / 2) % 8) of the row.
    auto read_a = [&](bf16x8 (&a)[4], const __bf16 *stage, int kq) __attribute__((always_inline)) {
        const uint32_t c = 4u * static_cast<uint32_t>(kq >> 1) + 2u * kh + static_cast<uint32_t>(kq & 1);
        const __bf16 *src = stage + grp * kTile + col * kStepK + 8u * (c ^ ((col >> 1) & 7u));
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(src + 32u * kStepK * i);
    };

    // One 64-k step = slices 4 odd .. 4 odd + 3 of half-block rc (odd = which
    // quarter of the half), read from stage cur. Slice kq's MFMAs run while
    // slice kq + 1 is read and decoded; during the last slice, the next step's
    // slice 0 is decoded (from rn when the next step starts a new half-block).
    // Slices 0 and 1 first issue the next step's activation loads (two
    // each); slices 1..3 of the first two steps of a block issue the next
    // block's weight loads (runs 0..10, then 11..21). Spread out like this,
    // the loads of eight wavefronts never pile up in front of the texture
    // unit at once.
    bf16x8 af[2][4], bf[2][2];
    auto step = [&](const __bf16 *cur, __bf16 *ahead, uint32_t s, int t, const GemmRaw &rc, const GemmRaw &rn,
                    uint32_t *wnext, uint32_t kbn) __attribute__((always_inline)) {
        const int odd = t & 1;
        read_a(af[0], cur, 0);
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            __builtin_amdgcn_sched_barrier(0);
            if (kq < 2) {
                dma_x(ahead, s + 1, 2u * kq);
                dma_x(ahead, s + 1, 2u * kq + 1u);
            }
            if (t < 2 && kq >= 1) {
                const uint32_t j0 = 11u * t + (kq == 1 ? 0u : kq == 2 ? 4u : 8u);
                const uint32_t nj = kq == 3 ? 3u : 4u;
#pragma unroll
                for (uint32_t j = 0; j < nj; ++j) dma_w(wnext, kbn, j0 + j);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kq < 3) {
                read_a(af[(kq + 1) & 1], cur, kq + 1);
                decode(rc, 4 * odd + kq + 1, bf[(kq + 1) & 1]);
            } else if (odd == 0) {
                decode(rc, 4, bf[0]);
            } else {
                decode(rn, 0, bf[0]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // A partial routing tile skips the row blocks it does not fill (their
                // rows are never stored). The dense path keeps every MFMA: the
                // branch cost it 2 us there.
                if (kRouted && i > 0 && 32u * i >= rows) continue;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kq & 1][i], bf[kq & 1][jj], acc[i][jj], 0, 0, 0);
            }
        }
    };

    // Block b of the group (K block kb0 + b) runs steps 4 b .. 4 b + 3 from
    // stages 0, 1, 0, 1 and weight buffer b % 2; its first two steps fill the
    // other weight buffer with block b + 1, which was last read in block
    // b - 1's first two steps. Raw bytes: half 1 of block b is read from LDS
    // in step 0 (used from the end of step 1), half 0 of block b + 1 in step 3
    // (used from the end of step 3). Step s stores step s + 1's activations
    // into stage (s + 1) % 2, last read in step s - 1. Barriers: each step
    // ends by waiting for its own activation loads; weight loads issued after
    // them may stay in flight, 11 after steps 0 and 1, none after steps 2 and
    // 3, so a block's weights are in before its predecessor's last step.
    GemmRaw raw[2];
#pragma unroll
    for (uint32_t j = 0; j < kWRuns; ++j) dma_w(ws0, kb0, j);
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) dma_x(xs0, 0, i);
    vm_barrier<0>();
    read_raw(raw[0], ws0, 0);
    decode(raw[0], 0, bf[0]);
    auto block = [&](uint32_t b, uint32_t *wcur, uint32_t *wnext) __attribute__((always_inline)) {
        const uint32_t kb = kb0 + b;
        const uint32_t s = 4u * b;
        read_raw(raw[1], wcur, 1);
        step(xs0, xs1, s, 0, raw[0], raw[1], wnext, kb + 1);
        __builtin_amdgcn_sched_barrier(0);
        vm_barrier<11>();
        __builtin_amdgcn_sched_barrier(0);
        step(xs1, xs0, s + 1, 1, raw[0], raw[1], wnext, kb + 1);
        __builtin_amdgcn_sched_barrier(0);
        vm_barrier<11>();
        __builtin_amdgcn_sched_barrier(0);
        step(xs0, xs1, s + 2, 2, raw[1], raw[0], wnext, kb + 1);
        __builtin_amdgcn_sched_barrier(0);
        vm_barrier<0>();
        __builtin_amdgcn_sched_barrier(0);
        read_raw(raw[0], wnext, 0);
        step(xs1, xs0, s + 3, 3, raw[1], raw[0], wnext, kb + 1);
        __builtin_amdgcn_sched_barrier(0);
        vm_barrier<0>();
        __builtin_amdgcn_sched_barrier(0);
    };
    // The missing last block of group 1 (odd block count) only keeps the
    // barrier count: four barriers, no loads, no MFMAs.
    auto idle = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 4; ++t) vm_barrier<0>();
    };
    uint32_t b = 0;
    for (; b + 2 <= nblk; b += 2) {
        block(b, ws0, ws1);
        if (kb0 + b + 1 < nb) block(b + 1, ws1, ws0);
        else idle();
    }
    if (b < nblk) {
        if (kb0 + b < nb) block(b, ws0, ws1);
        else idle();
    }

    // The two K halves meet: group 1 hands over row blocks 0 and 1, group 0
    // row blocks 2 and 3, lane-major (one dword per lane, rows of 64 lanes, a
    // 16 KiB region per wavefront in the stage and weight buffers). Both
    // groups add (lower half) + (upper half) in that order. The group index
    // selects register blocks only through uniform branches, so the
    // accumulators are never indexed at run time. The full barrier first
    // drains the loads still in flight (those past the group's range).
    __syncthreads();
    auto swap_of = [&](uint32_t wv2) -> float * {
        float *base = wv2 < 2 ? reinterpret_cast<float *>(xs0)
                              : (wv2 < 4 ? reinterpret_cast<float *>(xs1)
                                         : (wv2 < 6 ? reinterpret_cast<float *>(ws0) : reinterpret_cast<float *>(ws1)));
        return base + (wv2 & 1u) * 4096u;
    };
    float *const sw_mine = swap_of(wave);
    const float *const sw_other = swap_of(wave ^ 4u);
    auto give = [&](int base) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int v = 0; v < 16; ++v) sw_mine[(32u * ii + 16u * jj + v) * 64u + lane] = acc[base + ii][jj][v];
    };
    if (grp == 0) give(2);
    else give(0);
    __syncthreads();
    // D layout of a 32x32 tile: lane l holds column l % 32, rows 8(v/4) + 4(l/32) + v%4.
    const bool full = rows == kGM && n0 + kGN <= N;
    auto finish = [&](int base, bool lower_is_mine) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const uint32_t i = base + ii;
                const uint32_t n = n0 + 64u * wq + 32u * jj + col;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float other = sw_other[(32u * ii + 16u * jj + v) * 64u + lane];
                    const float mine = acc[base + ii][jj][v];
                    const float sum = lower_is_mine ? mine + other : other + mine;
                    const uint32_t m = 32u * i + 8u * (v >> 2) + 4u * kh + (v & 3);
                    const uint32_t dst = kRouted ? rowmap[m] : m0 + m;
                    // Non-temporal: 29 MB of y per M=512 call cannot stay in L2 anyway, and
                    // the streaming hint took about 1.5 us off the store phase at the end.
                    if (full || (m < rows && n < N))
                        __builtin_nontemporal_store(sum, &y[static_cast<uint64_t>(dst) * N + n]);
                }
                __builtin_amdgcn_sched_barrier(0);  // one 16-value group live at a time
            }
    };
    if (grp == 0) finish(0, true);
    else finish(2, false);
}

// k_gemv_seg in one shape over problems (grid y) problems: batch matrices, or routes from route0 when
// kRouted.
template <int M, uint32_t BW, int NI, bool kRouted>
void launch_seg(const float *x, const uint8_t *w, float *y, uint32_t N, uint32_t K, uint32_t problems,
                GemvBatch bt, GemvRoute rt, hipStream_t stream) {
    constexpr uint32_t rows = seg_rows(BW, NI);
    hipLaunchKernelGGL((k_gemv_seg<M, BW, NI, kRouted>), dim3((N + rows - 1) / rows, problems), dim3(64 * 16 / BW), 0,
                       stream, x, w, y, N, K, bt, rt);
}

// The large shape takes a launch once the small one would need more than one
// and a half rounds of workgroups on the chip for M = 1, more than one round
// for M = 2 (a round: the small shape's resident workgroups per CU, two for
// M = 1 and one for M = 2 at 113 and 186 VGPRs, times the CUs). Measured on
// one box, small against large shape (K = 4096 unless noted): M = 1 N = 8192
// 4.85 / 5.38 us, N = 12288 (1.5 rounds) 6.64 / 7.21, N = 14336 7.97 / 7.28,
// K = 8192 N = 8192 7.86 / 8.79, K = 2048 N = 14336 7.40 / 6.75, 3 x N = 4096
// 6.59 / 7.21; M = 2 N = 4096 (one round) 4.71 / 6.90, N = 6144 7.43 / 7.07,
// N = 8192 7.75 / 7.25, 2 x N = 4096 7.74 / 7.28.
template <int M>
bool seg_iters_large(uint32_t N, uint64_t problems) {
    static const uint64_t resident = [] {
        int n = 0, dev = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &n, reinterpret_cast<const void *>(k_gemv_seg<M, kSegSmallBW, kSegSmallNI, false>),
                64 * 16 / kSegSmallBW, 0) != hipSuccess || n < 1)
            n = 1;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        return static_cast<uint64_t>(n) * static_cast<uint64_t>(cus);
    }();
    constexpr uint32_t rows = seg_rows(kSegSmallBW, kSegSmallNI);
    const uint64_t wgs = static_cast<uint64_t>((N + rows - 1) / rows) * problems;
    return M == 1 ? 2 * wgs > 3 * resident : wgs > resident;
}

template <int M>
hipError_t launch_gemv_seg(const float *x, const uint8_t *w, float *y, uint32_t N, uint32_t K, uint32_t batches,
                           GemvBatch bt, hipStream_t stream) {
    if (seg_iters_large<M>(N, batches))
        launch_seg<M, kSegLargeBW, kSegLargeNI, false>(x, w, y, N, K, batches, bt, GemvRoute{}, stream);
    else
        launch_seg<M, kSegSmallBW, kSegSmallNI, false>(x, w, y, N, K, batches, bt, GemvRoute{}, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const uint8_t *blocks, uint64_t nblocks, float *out, hipStream_t stream) {
    const uint64_t waves = (nblocks + kRunBlocks - 1) / kRunBlocks;
    const uint64_t grid = (waves + 3) / 4;
    if (grid > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_dequantize, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, blocks,
                       reinterpret_cast<float4 *>(out), nblocks);
    return hipGetLastError();
}

hipError_t launch_gather(const uint8_t *table, const uint32_t *ids, float *out, uint32_t vocab,
                         uint32_t blocks_per_row, uint32_t n_tokens, int *status, int bad_value, hipStream_t stream) {
    const uint64_t runs = (blocks_per_row + kGatherRun - 1) / kGatherRun;
    const uint64_t grid = (static_cast<uint64_t>(n_tokens) * runs + 3) / 4;
    if (grid > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gather, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, table, ids,
                       reinterpret_cast<float4 *>(out), vocab, blocks_per_row, n_tokens, status, bad_value);
    return hipGetLastError();
}

hipError_t launch_gather_done(int *status, int seq, int *host_word, hipStream_t stream) {
    hipLaunchKernelGGL(k_gather_done, dim3(1), dim3(64), 0, stream, status, seq, host_word);
    return hipGetLastError();
}

hipError_t launch_gemv(const float *x, const uint8_t *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                       uint32_t batches, hipStream_t stream) {
    if (batches == 0 || batches > kMaxGridY) return hipErrorInvalidValue;
    const GemvBatch bt{static_cast<uint64_t>(M) * K, static_cast<uint64_t>(N) * (K / kQK) * kBlockBytes,
                       static_cast<uint64_t>(M) * N};
    switch (M) {
        case 1: return launch_gemv_seg<1>(x, w, y, N, K, batches, bt, stream);
        case 2: return launch_gemv_seg<2>(x, w, y, N, K, batches, bt, stream);
        case 3: case 4: case 5: case 6: case 7: case 8: {
            const uint32_t nb = K / kQK;
            const uint32_t wgs = (N + 16 * kMvTiles - 1) / (16 * kMvTiles);
            if (nb == kMvWaves) {
                hipLaunchKernelGGL(k_gemv_mfma_staged, dim3(wgs, batches), dim3(1024), 0, stream, x, w, y, M, N, bt);
            } else if (nb > kMvWaves) {
                hipLaunchKernelGGL(k_gemv_mfma_blocks, dim3(wgs, batches), dim3(1024), 0, stream, x, w, y, M, N, K, bt);
            } else {
                const uint32_t wpb = kMvWaves / nb;
                hipLaunchKernelGGL(k_gemv_mfma, dim3(wgs, batches), dim3(1024), 0, stream, x, w, y, M, N, K, bt,
                                   MvPlan{wpb, nb * wpb});
            }
            return hipGetLastError();
        }
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_mfma(const float *x, const uint8_t *w, float *y, uint32_t M, uint32_t N, uint32_t K,
                            void *x_bf16, hipStream_t stream) {
    const uint64_t n8 = static_cast<uint64_t>(M) * K / 8;
    const uint64_t want = (n8 + 256 * kXU - 1) / (256 * kXU);
    hipLaunchKernelGGL(k_x_to_bf16, dim3(static_cast<uint32_t>(want < 1024u ? want : 1024u)), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(x), static_cast<bf16x8 *>(x_bf16), n8);
    const uint32_t tiles_m = (M + kGM - 1) / kGM;
    const uint64_t tiles = static_cast<uint64_t>((N + kGN - 1) / kGN) * tiles_m;
    if (tiles > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gemm_q2k<false>, dim3(static_cast<uint32_t>(tiles)), dim3(512), 0, stream,
                       static_cast<const __bf16 *>(x_bf16), w, y, M, N, K, tiles_m, GemmRoute{});
    return hipGetLastError();
}

hipError_t launch_moe_gemv(const float *x, const uint8_t *w, const uint32_t *ids, float *y, uint32_t routes,
                           uint32_t x_div, uint32_t N, uint32_t K, uint32_t n_experts, uint64_t expert_stride,
                           int *status, hipStream_t stream) {
    const bool large = seg_iters_large<1>(N, routes);
    for (uint32_t r0 = 0; r0 < routes; r0 += kMaxGridY) {
        const uint32_t nr = routes - r0 < kMaxGridY ? routes - r0 : kMaxGridY;
        const GemvRoute rt{ids, status, expert_stride, r0, x_div, n_experts};
        if (large)
            launch_seg<1, kSegLargeBW, kSegLargeNI, true>(x, w, y, N, K, nr, GemvBatch{}, rt, stream);
        else
            launch_seg<1, kSegSmallBW, kSegSmallNI, true>(x, w, y, N, K, nr, GemvBatch{}, rt, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_moe_gemm(const uint8_t *w, float *y, uint32_t routes, uint32_t N, uint32_t K, uint32_t n_experts,
                           uint64_t expert_stride, MoeScratch s, hipStream_t stream) {
    const uint32_t tiles_m = moe_tiles_max(routes, n_experts);
    const uint64_t tiles = static_cast<uint64_t>((N + kGN - 1) / kGN) * tiles_m;
    if (tiles > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gemm_q2k<true>, dim3(static_cast<uint32_t>(tiles)), dim3(512), 0, stream,
                       static_cast<const __bf16 *>(s.x_bf16), w, y, routes, N, K, tiles_m,
                       GemmRoute{s.tiles, s.perm, expert_stride});
    return hipGetLastError();
}

}  // namespace q2k
