"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Rules (the page is the docs.rs source page of mlx-native 0.10.8,
tests/deepseek_q2_k.rs):
  * dequantize and gather: bit-identical (the decoded value is unique);
  * fp32 GEMV (M <= 8): |y - exact| <= 1e-5 * sum|x*w|, and the page's own
    2e-4 absolute bound on its run_dense(1) fixture;
  * bf16 matrix-core path (M > 8): |y - exact| <= 4e-3 * sum|x*w| + 1e-6,
    plus |y - exact_bf16| <= K * 2^-24 * sum|bf16(x)*bf16(w)| + 1e-6 against
    the oracle run on bf16-rounded operands (fp32 accumulation error bound);
  * one-hot activations pin single weights bit for bit (bf16-rounded, ties to
    even, on the matrix-core path).
Inputs are the seeded workloads of synth.CONFIGS and the page fixtures.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import ggml_q2_dequant_amd as q2k  # noqa: E402

pytestmark = pytest.mark.gpu

QK_K, BB = 256, 84
GEMV_REL = 1e-5
MFMA_REL, MFMA_ABS = 4e-3, 1e-6


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q2k.load_library()
    yield torch.device("cuda:0")
    torch.cuda.synchronize()


_inputs = {}


def inputs(i):
    if i not in _inputs:
        _inputs[i] = synth.make_inputs(i)
    return _inputs[i]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def gpu_dequantize(blocks):
    b = dev(blocks)
    out = torch.empty(blocks.size // BB * QK_K, dtype=torch.float32, device="cuda:0")
    q2k.q2k_dequantize(b, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_matmul(x, blocks, M, N, K, path=q2k.PATH_AUTO):
    xd, wd = dev(x.astype(np.float32)), dev(blocks)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    q2k.q2k_matmul_path(xd, wd, y, M, N, K, path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_gather(table, ids, vocab, dim, nt):
    out = torch.full((nt, dim), float("nan"), dtype=torch.float32, device="cuda:0")
    q2k.q2k_embedding_gather(dev(table), dev(np.asarray(ids, dtype=np.uint32)), out, vocab, dim, nt)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def bits_equal(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return a.shape == b.shape and np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def check_gemv(y, x, blocks, M, N, K):
    ref, a = oracle.matmul(x, blocks, M, N, K, nthreads=oracle.host_threads())
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(np.isfinite(y))
    worst = float(np.max(err / np.maximum(a, 1e-300)))
    assert np.all(err <= GEMV_REL * a), "max |err|/A = %g" % worst
    return worst


def check_mfma(y, x, blocks, M, N, K, nthreads=None):
    nthreads = nthreads or oracle.host_threads()
    ref, a = oracle.matmul(x, blocks, M, N, K, nthreads=nthreads)
    refb, ab = oracle.matmul(x, blocks, M, N, K, bf16_operands=True, nthreads=nthreads)
    assert np.all(np.isfinite(y))
    y64 = y.astype(np.float64)
    err = np.abs(y64 - ref)
    assert np.all(err <= MFMA_REL * a + MFMA_ABS), "max |err|/A = %g" % float(np.max(err / a))
    errb = np.abs(y64 - refb)
    assert np.all(errb <= K * 2.0 ** -24 * ab + MFMA_ABS), "max |err_bf16|/A = %g" % float(np.max(errb / ab))
    return float(np.max(err / a))


# ----------------------------------------------------------------- dequantize

def test_dequantize_page_fixture_blocks_bitwise():
    blocks = np.concatenate([synth.page_block(s) for s in range(256)])
    assert bits_equal(gpu_dequantize(blocks), oracle.dequantize(blocks))


def test_dequantize_config0_blocks_bitwise():
    blocks = inputs(0).blocks
    assert bits_equal(gpu_dequantize(blocks), oracle.dequantize(blocks))


def _with_d(blk, d_bits, dmin_bits):
    blk = blk.copy()
    blk[80], blk[81], blk[82], blk[83] = d_bits & 255, d_bits >> 8, dmin_bits & 255, dmin_bits >> 8
    return blk


def test_dequantize_special_d_dmin_bitwise():
    rng = np.random.Generator(np.random.PCG64(31))
    base = synth.random_blocks(rng, 1)
    specials = [0x0000, 0x8000, 0x0001, 0x03FF, 0x8001, 0x0400, 0x3C00, 0xBC00, 0x7BFF, 0xFBFF,
                0x7C00, 0xFC00, 0x7E00, 0x2E66, 0x1234]
    blocks = np.concatenate([_with_d(base, d, m) for d in specials for m in specials])
    assert bits_equal(gpu_dequantize(blocks), oracle.dequantize(blocks))


def test_dequantize_random_bytes_all_patterns_bitwise():
    # Fully random bytes (any f16 in d/dmin, any nibble) over 4099 blocks.
    rng = np.random.Generator(np.random.PCG64(32))
    blocks = rng.integers(0, 256, 4099 * BB, dtype=np.uint8)
    assert bits_equal(gpu_dequantize(blocks), oracle.dequantize(blocks))


def test_dequantize_large_buffer_grid_stride_bitwise():
    # More blocks than one grid of the kernel covers, so the grid-stride loop runs.
    rng = np.random.Generator(np.random.PCG64(33))
    nb = 262144 + 37
    blocks = synth.random_blocks(rng, nb)
    assert bits_equal(gpu_dequantize(blocks), oracle.dequantize(blocks))


def test_dequantize_rejects_page_malformed_buffers_on_device():
    blk = dev(synth.page_block(1))
    out = torch.empty(QK_K, dtype=torch.float32, device="cuda:0")
    with pytest.raises(q2k.Q2KInvalidArgument):
        q2k.q2k_dequantize(blk, out, blocks_bytes=BB - 1)
    with pytest.raises(q2k.Q2KInvalidArgument):
        q2k.q2k_dequantize(blk, out, out_elems=QK_K - 1)


# ----------------------------------------------------------------- gather

def test_gather_page_fixture_and_bad_id():
    vocab = 3
    table = np.concatenate([synth.page_block(r + 2) for r in range(vocab)])
    got = gpu_gather(table, [2, 0], vocab, QK_K, 2)
    want = oracle.gather(table, [2, 0], vocab, QK_K, 2)
    assert bits_equal(got, want)
    assert np.all(np.abs(got - want) <= 1e-6)  # the page's own bound
    with pytest.raises(q2k.Q2KIdOutOfRange):
        gpu_gather(table, [2, vocab], vocab, QK_K, 2)
    with pytest.raises(q2k.Q2KIdOutOfRange):
        gpu_gather(table, [0xFFFFFFFF, 1], vocab, QK_K, 2)
    # A good call after a rejected one succeeds (the status word is cleared).
    assert bits_equal(gpu_gather(table, [1, 1], vocab, QK_K, 2), oracle.gather(table, [1, 1], vocab, QK_K, 2))


def test_gather_returns_after_work_queued_ahead_of_it():
    # The call returns only once everything queued on its stream before it has
    # ended: with a short queue (it polls the word its completion kernel
    # publishes) and behind a spin of many milliseconds (past the poll bound it
    # waits on the stream). A rejected id between good calls must not leak into
    # the next call's verdict.
    vocab = 3
    table = np.concatenate([synth.page_block(r + 2) for r in range(vocab)])
    tbl = dev(table)
    s = torch.cuda.current_stream()
    marker = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    cases = [(0, [2, 0]), (20_000_000, [1, 2]), (0, [0, 0]), (0, [2, vocab]), (20_000_000, [1, 0]), (0, [vocab + 7, 1]),
             (0, [1, 1])]
    for k, (cycles, ids) in enumerate(cases):
        out = torch.full((2, QK_K), float("nan"), dtype=torch.float32, device="cuda:0")
        idd = dev(np.asarray(ids, dtype=np.uint32))
        torch.cuda.synchronize()
        if cycles:
            torch.cuda._sleep(cycles)
        marker.fill_(float(k + 1))
        ev = torch.cuda.Event()
        ev.record(s)
        if max(ids) >= vocab:
            with pytest.raises(q2k.Q2KIdOutOfRange):
                q2k.q2k_embedding_gather(tbl, idd, out, vocab, QK_K, 2, stream=s)
            assert ev.query(), "returned before the work queued ahead ended"
            continue
        q2k.q2k_embedding_gather(tbl, idd, out, vocab, QK_K, 2, stream=s)
        assert ev.query(), "returned before the work queued ahead ended"
        assert float(marker.item()) == float(k + 1)
        assert bits_equal(out.cpu().numpy(), oracle.gather(table, ids, vocab, QK_K, 2))


def test_gather_ragged_multi_block_rows_with_duplicates():
    rng = np.random.Generator(np.random.PCG64(34))
    vocab, dim = 5, 768
    table = synth.random_blocks(rng, vocab * dim // QK_K)
    ids = [4, 4, 0, 2, 3, 1, 4]
    assert bits_equal(gpu_gather(table, ids, vocab, dim, len(ids)), oracle.gather(table, ids, vocab, dim, len(ids)))


def test_gather_rows_longer_than_one_run():
    # 70 blocks per row: 17 runs of 4 blocks and a ragged run of 2 per token.
    rng = np.random.Generator(np.random.PCG64(38))
    vocab, dim = 3, 70 * QK_K
    table = synth.random_blocks(rng, vocab * dim // QK_K)
    ids = [2, 0, 1, 2, 0]
    assert bits_equal(gpu_gather(table, ids, vocab, dim, len(ids)), oracle.gather(table, ids, vocab, dim, len(ids)))
    with pytest.raises(q2k.Q2KIdOutOfRange):
        gpu_gather(table, [1, vocab, 0], vocab, dim, 3)


def test_gather_config2_full_size_and_bad_id():
    inp = inputs(2)
    c = inp.config
    table = dev(inp.blocks)
    ids = dev(inp.ids)
    out = torch.full((c.n_tokens, c.embed_dim), float("nan"), dtype=torch.float32, device="cuda:0")
    q2k.q2k_embedding_gather(table, ids, out, c.vocab, c.embed_dim, c.n_tokens)
    torch.cuda.synchronize()
    want = oracle.gather(inp.blocks, inp.ids, c.vocab, c.embed_dim, c.n_tokens, nthreads=oracle.host_threads())
    assert bits_equal(out.cpu().numpy(), want)

    bad = synth.bad_ids(inp)
    out.fill_(float("nan"))
    with pytest.raises(q2k.Q2KIdOutOfRange):
        q2k.q2k_embedding_gather(table, dev(bad), out, c.vocab, c.embed_dim, c.n_tokens)
    got = out.cpu().numpy()
    keep = np.arange(c.n_tokens) != c.bad_id_pos
    assert bits_equal(got[keep], want[keep])      # valid rows are still written
    assert np.all(np.isnan(got[c.bad_id_pos]))    # the bad row is never touched


def test_gather_async_matches_the_gather_and_reports_bad_ids():
    # The asynchronous gather writes the same rows; a bad id sets the caller's
    # status word (which no later call clears) and leaves its row untouched.
    rng = np.random.Generator(np.random.PCG64(39))
    vocab, dim, nt = 300, 1280, 40
    table_h = synth.random_blocks(rng, vocab * dim // QK_K)
    ids_h = rng.integers(0, vocab, nt).astype(np.uint32)
    ids_h[5] = ids_h[9]
    table, status = dev(table_h), torch.zeros(1, dtype=torch.int32, device="cuda:0")
    out = torch.full((nt, dim), float("nan"), dtype=torch.float32, device="cuda:0")
    q2k.q2k_embedding_gather_async(table, dev(ids_h), out, vocab, dim, nt, status)
    torch.cuda.synchronize()
    want = oracle.gather(table_h, ids_h, vocab, dim, nt)
    assert bits_equal(out.cpu().numpy(), want) and int(status.item()) == 0
    assert bits_equal(gpu_gather(table_h, ids_h, vocab, dim, nt), out.cpu().numpy())

    bad = ids_h.copy()
    bad[[3, 17]] = [vocab, 0xFFFFFFFF]
    out.fill_(float("nan"))
    q2k.q2k_embedding_gather_async(table, dev(bad), out, vocab, dim, nt, status)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    keep = np.ones(nt, bool)
    keep[[3, 17]] = False
    assert int(status.item()) == 1
    assert bits_equal(got[keep], want[keep]) and np.all(np.isnan(got[~keep]))
    q2k.q2k_embedding_gather_async(table, dev(ids_h), out, vocab, dim, nt, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1 and bits_equal(out.cpu().numpy(), want)


def test_gather_last_row_of_table():
    inp = inputs(2)
    c = inp.config
    ids = np.array([c.vocab - 1, 0, c.vocab - 1], dtype=np.uint32)
    got = gpu_gather(inp.blocks, ids, c.vocab, c.embed_dim, 3)
    assert bits_equal(got, oracle.gather(inp.blocks, ids, c.vocab, c.embed_dim, 3))


# ----------------------------------------------------------------- GEMV (M <= 8)

def test_gemv_page_run_dense_rows1():
    blocks = np.concatenate([synth.page_block(r + 1) for r in range(8)])
    x = synth.page_input(1).reshape(1, QK_K)
    y = gpu_matmul(x, blocks, 1, 8, QK_K)
    want = oracle.matmul_f32seq(x, blocks, 1, 8, QK_K)
    assert np.all(np.abs(y - want) <= 2e-4)        # the page's tolerance
    check_gemv(y, x, blocks, 1, 8, QK_K)


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_gemv_configs(cfg):
    inp = inputs(cfg)
    c = inp.config
    y = gpu_matmul(inp.x, inp.blocks, c.M, c.N, c.K)
    worst = check_gemv(y, inp.x, inp.blocks, c.M, c.N, c.K)
    print("parity cfg%d (%s): max |y - y_ref| / A = %.3g" % (cfg, c.name, worst))


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (3, 7, 768), (8, 130, 1280), (5, 4097, 256), (2, 9, 4352),
                                   (7, 33, 1024), (8, 100, 8448), (4, 65, 4352)])
def test_gemv_ragged_shapes(M, N, K):
    # For 3 <= M <= 8, K < 4096 gives blocks shared by several wavefronts, and
    # K > 4096 (33 and 17 blocks here) wavefronts that walk several blocks.
    rng = np.random.Generator(np.random.PCG64(M * 1000 + N + K))
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y = gpu_matmul(x, blocks, M, N, K)
    check_gemv(y, x, blocks, M, N, K)


@pytest.mark.parametrize("M,N,K", [(1, 40001, 1024), (2, 33333, 768), (1, 70003, 4096), (2, 9999, 3840),
                                   (1, 5, 256), (2, 4, 512), (1, 14336, 4096), (2, 16384, 4096), (2, 6144, 4096)])
def test_gemv_large_ragged_launches(M, N, K):
    # M <= 2 launches with many rows take the large chunked shape (32 rows per
    # workgroup, in row groups of 4): large ragged N
    # leaves a partial last workgroup and group; K below 4096 a partial chunk.
    rng = np.random.Generator(np.random.PCG64(M * 7 + N + K))
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y = gpu_matmul(x, blocks, M, N, K)
    check_gemv(y, x, blocks, M, N, K)
    if M == 2:
        for m in range(2):
            assert bits_equal(gpu_matmul(x[m:m + 1], blocks, 1, N, K), y[m:m + 1])


@pytest.mark.parametrize("M", [1, 2])
def test_gemv_large_and_small_shapes_agree_bitwise(M):
    # A large launch runs the chunked kernel's large shape (four wavefronts of
    # four blocks); a 4096-row call the small one (eight wavefronts of two).
    # Both run the same per-lane arithmetic and summation order, so the shared
    # rows must match bit for bit (that is what keeps routed and batched rows
    # equal to single calls).
    N, K, n_small = 40000, 4096, 4096
    rng = np.random.Generator(np.random.PCG64(4200 + M))
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y_big = gpu_matmul(x, blocks, M, N, K)
    y_small = gpu_matmul(x, blocks[:n_small * (K // QK_K) * BB], M, n_small, K)
    assert bits_equal(y_big[:, :n_small], y_small)
    check_gemv(y_small, x, blocks[:n_small * (K // QK_K) * BB], M, n_small, K)


@pytest.mark.parametrize("M", [3, 8])
def test_gemv_wide_dynamic_range_activations(M):
    # 3 <= M <= 8 splits each row of each 256-column block into two f16 pieces
    # after a power-of-two scale of that row and block: rows far apart in
    # magnitude, a 1e3 spread inside blocks, zero rows and exact zeros must
    # all stay within the fp32 rule.
    rng = np.random.Generator(np.random.PCG64(36 + M))
    N, K = 300, 1280
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.float32(10.0) ** rng.integers(-3, 4, (M, K)).astype(np.float32)   # 1e3 spread within rows
    scales = np.array([1e-20, 1.0, 1e20, 0.0, 3e-5, 7e8, 1.0, 2.0 ** -60], np.float32)[:M]
    x *= scales[:, None]
    x[0, ::7] = 0.0
    y = gpu_matmul(x, blocks, M, N, K)
    zero = scales == 0
    assert np.all(y[zero] == 0.0)
    check_gemv(y[~zero], x[~zero], blocks, int((~zero).sum()), N, K)


def test_gemv_rows_do_not_depend_on_other_rows():
    # An output row depends only on its own activation row: rows of a call
    # equal the same rows computed in a call of the same kernel variant
    # (M <= 2 and 3 <= M <= 8 use different kernels) with other companions.
    inp = inputs(3)
    c = inp.config
    y8 = gpu_matmul(inp.x, inp.blocks, 8, c.N, c.K)
    y3 = gpu_matmul(inp.x[2:5], inp.blocks, 3, c.N, c.K)
    assert bits_equal(y3, y8[2:5])
    perm = [7, 0, 5, 1, 6, 2, 4, 3]
    assert bits_equal(gpu_matmul(inp.x[perm], inp.blocks, 8, c.N, c.K), y8[perm])
    y2 = gpu_matmul(inp.x[3:5], inp.blocks, 2, c.N, c.K)
    for m in range(2):
        assert bits_equal(gpu_matmul(inp.x[3 + m:4 + m], inp.blocks, 1, c.N, c.K), y2[m:m + 1])


@pytest.mark.parametrize("M,path", [(1, q2k.PATH_GEMV), (2, q2k.PATH_GEMV), (8, q2k.PATH_GEMV), (9, q2k.PATH_MFMA)])
def test_largest_k_every_path(M, path):
    # K at the library's limit (2^21, 8192 blocks a row): the longest walks
    # over K and the largest per-workgroup offsets any call can reach, on a
    # ragged N.
    K, N = 1 << 21, 17
    rng = np.random.Generator(np.random.PCG64(2100 + M))
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y = gpu_matmul(x, blocks, M, N, K, path)
    worst = (check_gemv if path == q2k.PATH_GEMV else check_mfma)(y, x, blocks, M, N, K)
    print("K = 2^21, M=%d: max |y - y_ref| / A = %.3g" % (M, worst))


def test_gemv_one_hot_returns_weights_bitwise():
    rng = np.random.Generator(np.random.PCG64(35))
    N, K = 40, 1024
    blocks = synth.random_blocks(rng, N * K // QK_K)
    dense = oracle.dequantize(blocks).reshape(N, K)
    for ks in ([0, 1, 15, 16, 31, 32, 127, 128], [255, 256, 511, 512, 700, 1000, 1022, 1023]):
        x = np.zeros((len(ks), K), dtype=np.float32)
        x[np.arange(len(ks)), ks] = 1.0
        y = gpu_matmul(x, blocks, len(ks), N, K)
        assert bits_equal(y, dense[:, ks].T)


def test_gemv_is_deterministic():
    inp = inputs(1)
    c = inp.config
    a = gpu_matmul(inp.x, inp.blocks, c.M, c.N, c.K)
    b = gpu_matmul(inp.x, inp.blocks, c.M, c.N, c.K)
    assert bits_equal(a, b)


# ----------------------------------------------------------------- batched mat-vec

def gpu_matmul_batched(x, blocks, batches, M, N, K):
    xd, wd = dev(np.ascontiguousarray(x, dtype=np.float32)), dev(blocks)
    y = torch.full((batches, M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    q2k.q2k_matmul_batched(xd, wd, y, batches, M, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_batched_page_fixture_equals_independent_calls_bytewise():
    # The page's batched mat-vec test: 3 matrices of 8 rows, K = 256, block(b*8 + row + 1),
    # input(3) split one row per matrix; batched output equals serial M = 1 calls byte for byte.
    batches, n = 3, 8
    blocks = np.concatenate([synth.page_block(b * n + r + 1) for b in range(batches) for r in range(n)])
    x = synth.page_input(batches).reshape(batches, 1, QK_K)
    yb = gpu_matmul_batched(x, blocks, batches, 1, n, QK_K)
    per = n * BB
    for b in range(batches):
        ys = gpu_matmul(x[b], blocks[b * per:(b + 1) * per], 1, n, QK_K)
        assert bits_equal(yb[b], ys)
    ref, a = oracle.matmul_batched(x, blocks, batches, 1, n, QK_K)
    assert np.all(np.abs(yb - ref) <= GEMV_REL * a)
    for b in range(batches):
        assert np.all(np.abs(yb[b] - oracle.matmul_f32seq(x[b], blocks[b * per:(b + 1) * per], 1, n, QK_K)) <= 2e-4)


# The last two stacks are large enough for the large chunked shape, while each single call runs the small
# one: the batched rows must still equal the single calls bit for bit.
@pytest.mark.parametrize("batches,M,N,K", [(2, 1, 130, 768), (5, 2, 33, 256), (3, 3, 70, 1280), (4, 8, 257, 512),
                                           (1, 5, 4097, 256), (6, 7, 9, 4352), (8, 1, 4096, 512), (4, 2, 2048, 512)])
def test_batched_equals_independent_calls_and_oracle(batches, M, N, K):
    rng = np.random.Generator(np.random.PCG64(batches * 100003 + M * 1009 + N * 31 + K))
    blocks = synth.random_blocks(rng, batches * N * K // QK_K)
    x = rng.standard_normal((batches, M, K), dtype=np.float32)
    yb = gpu_matmul_batched(x, blocks, batches, M, N, K)
    per = N * K // QK_K * BB
    for b in range(batches):
        assert bits_equal(yb[b], gpu_matmul(x[b], blocks[b * per:(b + 1) * per], M, N, K))
    ref, a = oracle.matmul_batched(x, blocks, batches, M, N, K, nthreads=oracle.host_threads())
    assert np.all(np.abs(yb.astype(np.float64) - ref) <= GEMV_REL * a)


def test_batched_more_problems_than_one_launch_covers():
    # 65 537 one-row problems: the library splits them over two launches.
    batches, M, N, K = 65537, 1, 1, 256
    rng = np.random.Generator(np.random.PCG64(41))
    blocks = synth.random_blocks(rng, batches)
    x = rng.uniform(-1, 1, (batches, M, K)).astype(np.float32)
    yb = gpu_matmul_batched(x, blocks, batches, M, N, K)
    ref, a = oracle.matmul_batched(x, blocks, batches, M, N, K)
    assert np.all(np.abs(yb.astype(np.float64) - ref) <= GEMV_REL * a)
    for b in (0, 1, 65534, 65535, 65536):
        assert bits_equal(yb[b], gpu_matmul(x[b], blocks[b * BB:(b + 1) * BB], M, N, K))


def test_batched_rejects_m_above_eight_on_device():
    with pytest.raises(q2k.Q2KInvalidArgument):
        gpu_matmul_batched(np.zeros((2, 9, QK_K), np.float32), np.zeros(2 * BB, np.uint8), 2, 9, 1, QK_K)


# ----------------------------------------------------------------- matrix-core path (M > 8)

def test_mfma_page_run_dense_rows9_relative_rule():
    # The page's prefill fixture (9 rows, 8 weight rows, K = 256). Its 1e-2
    # absolute bound assumes a kernel keeping more than bf16 precision; the
    # bf16 path is held to the relative rule instead.
    blocks = np.concatenate([synth.page_block(r + 1) for r in range(8)])
    x = synth.page_input(9).reshape(9, QK_K)
    y = gpu_matmul(x, blocks, 9, 8, QK_K)
    check_mfma(y, x, blocks, 9, 8, QK_K)


def test_mfma_forced_on_config0():
    inp = inputs(0)
    c = inp.config
    y = gpu_matmul(inp.x, inp.blocks, c.M, c.N, c.K, path=q2k.PATH_MFMA)
    check_mfma(y, inp.x, inp.blocks, c.M, c.N, c.K)


@pytest.mark.parametrize("M,N,K", [(9, 8, 256), (64, 64, 512), (100, 130, 768), (129, 257, 1280),
                                   (256, 384, 4096), (17, 1000, 2304)])
def test_mfma_ragged_shapes(M, N, K):
    rng = np.random.Generator(np.random.PCG64(M * 7919 + N * 31 + K))
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y = gpu_matmul(x, blocks, M, N, K)
    check_mfma(y, x, blocks, M, N, K)


def test_mfma_config4_full_size_every_output():
    # The full M=512, N=14336, K=4096 launch (224 workgroups in the XCD-banded
    # tile order), every one of its 7 340 032 outputs against the f64 oracle and
    # the oracle on bf16-rounded operands.
    import time
    inp = inputs(4)
    c = inp.config
    y = gpu_matmul(inp.x, inp.blocks, c.M, c.N, c.K)
    t0 = time.perf_counter()
    worst = check_mfma(y, inp.x, inp.blocks, c.M, c.N, c.K)
    print("parity cfg4 (%s, all %d outputs): max |y - y_ref| / A = %.3g (oracle %.1f s on %d threads)" % (
        c.name, c.M * c.N, worst, time.perf_counter() - t0, oracle.host_threads()))


@pytest.mark.parametrize("M,N,K", [(256, 1024, 512), (512, 1024, 1024), (384, 2048, 512), (200, 1000, 768),
                                   (1000, 520, 256)])
def test_mfma_xcd_banded_tile_order_every_output(M, N, K):
    # Tile counts that are multiples of 8 (2x4, 4x4, 3x8, ragged 2x4, ragged 8x3)
    # take the XCD-banded block-to-tile order; every output is compared.
    tiles = ((M + 127) // 128) * ((N + 255) // 256)
    assert tiles % 8 == 0
    rng = np.random.Generator(np.random.PCG64(M * 31 + N * 7 + K))
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y = gpu_matmul(x, blocks, M, N, K)
    check_mfma(y, x, blocks, M, N, K)


def test_mfma_non_finite_scales_give_nan_columns():
    # d = +inf with zero scale nibbles and zero codes makes every d*sc*q - dmin*mn NaN (inf * 0),
    # even for q = 0, and dmin = NaN makes the whole block NaN: those columns of y are NaN, the
    # rest match the oracle.
    rng = np.random.Generator(np.random.PCG64(39))
    M, N, K = 9, 16, 512
    blocks = synth.random_blocks(rng, N * K // QK_K).reshape(N, K // QK_K, BB).copy()
    blocks[3, 0, 0:16] &= 0xF0                                                  # scales 0
    blocks[3, 0, 16:80] = 0                                                     # codes 0
    blocks[3, 0, 80:82] = np.frombuffer(np.float16(np.inf).tobytes(), np.uint8)  # d = +inf
    blocks[7, 1, 82:84] = np.frombuffer(np.float16(np.nan).tobytes(), np.uint8)  # dmin = NaN
    blocks = blocks.reshape(-1)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y = gpu_matmul(x, blocks, M, N, K)
    ref, _ = oracle.matmul(x, blocks, M, N, K)
    assert np.array_equal(np.isnan(y), np.isnan(ref)) and np.all(np.isnan(y[:, [3, 7]]))
    keep = [n for n in range(N) if n not in (3, 7)]
    check_mfma(y[:, keep], x, synth.rows_of(blocks, K, keep), M, len(keep), K)


def test_mfma_one_hot_returns_bf16_weights_bitwise():
    rng = np.random.Generator(np.random.PCG64(37))
    N, K = 72, 1024
    blocks = synth.random_blocks(rng, N * K // QK_K)
    dense = oracle.dequantize(blocks).reshape(N, K)
    ks = [0, 1, 15, 16, 31, 32, 127, 128, 255, 256, 511, 512, 700, 1000, 1022, 1023]
    x = np.zeros((len(ks), K), dtype=np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    y = gpu_matmul(x, blocks, len(ks), N, K)
    assert bits_equal(y, oracle.bf16_round(dense[:, ks].T).reshape(len(ks), N))


def _identity_blocks(N, K):
    """W[n, k] = 1 if k == n else 0: d = 1, scale nibble 1, min 0, one code 1."""
    nb = K // QK_K
    blocks = np.zeros((N, nb, BB), dtype=np.uint8)
    blocks[:, :, 0:16] = 0x01
    blocks[:, :, 80:82] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    for n in range(N):
        kb, e = divmod(n, QK_K)
        byte = 32 * (e // 128) + e % 32
        blocks[n, kb, 16 + byte] = 1 << (2 * ((e // 32) % 4))
    return blocks.reshape(-1)


def test_mfma_rounds_activations_to_nearest_even():
    N, K, M = 16, 256, 12
    blocks = _identity_blocks(N, K)
    dense = oracle.dequantize(blocks).reshape(N, K)
    assert np.array_equal(dense[:, :N], np.eye(N, dtype=np.float32))
    ulp = 2.0 ** -7
    ties = np.array([1 + ulp / 2, 1 + 3 * ulp / 2, -(1 + ulp / 2), 3 + 3 * ulp, 1 + ulp / 2 + 2.0 ** -20,
                     2.0 ** -100 * (1 + ulp / 2)], dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(38))
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[: len(ties), 0] = ties
    y = gpu_matmul(x, blocks, M, N, K)
    assert bits_equal(y, oracle.bf16_round(x[:, :N]).reshape(M, N))


def test_mfma_is_deterministic():
    rng = np.random.Generator(np.random.PCG64(39))
    M, N, K = 200, 300, 1024
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    assert bits_equal(gpu_matmul(x, blocks, M, N, K), gpu_matmul(x, blocks, M, N, K))


# ----------------------------------------------------------------- measurement aid

def test_read_probe_reads_every_word():
    # libq2k_probe (the benchmark's plain-read kernel, not part of the C ABI) stores one XOR word per
    # workgroup; their XOR is the XOR of all data words, for every launch shape the benchmark sweeps.
    import ctypes
    from ggml_q2_dequant_amd import build
    probe = ctypes.CDLL(build.PROBE_LIB)
    probe.q2k_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    probe.q2k_probe_read.restype = ctypes.c_int
    rng = np.random.Generator(np.random.PCG64(44))
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda:0")
    for nbytes in (16, 4096 + 16, 5 * 1024 * 1024 + 48):
        data = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
        d = dev(data.view(np.int32))
        for grid, unroll in ((0, 4), (256, 1), (2048, 16), (16384, 2), (7, 8)):
            sink.zero_()
            rc = probe.q2k_probe_read(d.data_ptr(), nbytes, sink.data_ptr(), sink.numel(), grid, unroll,
                                      torch.cuda.current_stream().cuda_stream)
            assert rc == 0
            torch.cuda.synchronize()
            got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
            assert got == np.bitwise_xor.reduce(data), (nbytes, grid, unroll)
    assert probe.q2k_probe_read(d.data_ptr(), 20, sink.data_ptr(), sink.numel(), 0, 4, None) == 1
    assert probe.q2k_probe_read(d.data_ptr(), 64, sink.data_ptr(), 8, 16, 4, None) == 1
    assert probe.q2k_probe_read(d.data_ptr(), 64, sink.data_ptr(), sink.numel(), 0, 3, None) == 1


# ----------------------------------------------------------------- the fp32 GEMV's error bound at its edges

def _code_min_magnitudes(blocks, N, K):
    """Per weight: |d*sc*q| and |dmin*mn| (f64), from the Q2_K record layout (scales @0, codes @16, d @80, dmin @82)."""
    b = np.asarray(blocks, np.uint8).reshape(N, K // QK_K, BB)
    d = b[:, :, 80:82].copy().view(np.float16)[:, :, 0].astype(np.float64)
    dmin = b[:, :, 82:84].copy().view(np.float16)[:, :, 0].astype(np.float64)
    e = np.arange(QK_K)
    sbyte = b[:, :, e // 16].astype(np.int64)
    code = (b[:, :, 16 + 32 * (e // 128) + e % 32].astype(np.int64) >> (2 * ((e // 32) % 4))) & 3
    codes = np.abs(d[:, :, None] * (sbyte & 15) * code).reshape(N, K)
    mins = np.abs(dmin[:, :, None] * (sbyte >> 4)).reshape(N, K)
    return codes, mins


def _b_bound(x, blocks, M, N, K):
    """B[m, n] = sum_k |x[m, k]| * (|d*sc*q| + |dmin*mn|): what the M <= 2 kernels' error is relative to."""
    codes, mins = _code_min_magnitudes(blocks, N, K)
    return np.abs(np.asarray(x, np.float64)).reshape(M, K) @ (codes + mins).T


def _m2_bound(K):
    return (27 + 2 * ((K + 4095) // 4096)) * 2.0 ** -24


def _m8_bound(x, blocks, M, N, K):
    """The 3 <= M <= 8 bound: 2^-18 B + 2^-6 sum_b max_k|x| (max_k |d*sc*q| + 16 max_s |dmin*mn|)."""
    codes, mins = _code_min_magnitudes(blocks, N, K)
    nb = K // QK_K
    xmax = np.abs(np.asarray(x, np.float64)).reshape(M, nb, QK_K).max(axis=2)              # [M, blocks]
    wmax = codes.reshape(N, nb, QK_K).max(axis=2) + 16 * mins.reshape(N, nb, QK_K).max(axis=2)  # [N, blocks]
    return 2.0 ** -18 * _b_bound(x, blocks, M, N, K) + 2.0 ** -6 * xmax @ wmax.T


def _block(d, dmin, scale_byte, code_byte):
    blk = np.zeros(BB, np.uint8)
    blk[0:16] = scale_byte
    blk[16:80] = code_byte
    blk[80:82] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
    blk[82:84] = np.frombuffer(np.float16(dmin).tobytes(), np.uint8)
    return blk


@pytest.mark.parametrize("M", [1, 2])
def test_gemv_blocks_whose_weights_cancel_to_zero(M):
    # d*sc*q == dmin*mn for every element (d = dmin = 1, sc = mn = 2, every code 1, or sc = 1, mn = 3, every code 3):
    # each weight is exactly 0, so sum |x*w| = 0, but the factored form d*sum(sc*q*x) - dmin*sum(mn*x) rounds its
    # two sums separately. The result must stay within the stated bound against B, which is not zero.
    rng = np.random.Generator(np.random.PCG64(4400 + M))
    N, K = 24, 1024
    zero_a = _block(1.0, 1.0, 0x22, 0x55)   # sc 2, mn 2, codes 1
    zero_b = _block(0.5, 0.5, 0x31, 0xFF)   # sc 1, mn 3, codes 3: d*1*3 = dmin*3
    blocks = np.concatenate([zero_a if (i + j) % 2 else zero_b for i in range(N) for j in range(K // QK_K)])
    assert np.all(oracle.dequantize(blocks) == 0.0)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y = gpu_matmul(x, blocks, M, N, K)
    b = _b_bound(x, blocks, M, N, K)
    assert np.all(b > 0)
    assert np.all(np.abs(y.astype(np.float64)) <= _m2_bound(K) * b), "max |y| / B = %g" % np.max(np.abs(y) / b)
    print("weights all zero, M=%d: max |y| / B = %.3g (bound %.3g)" % (M, np.max(np.abs(y) / b), _m2_bound(K)))


@pytest.mark.parametrize("M", [1, 2])
def test_gemv_near_cancelling_blocks_within_the_stated_bound(M):
    # Random blocks whose min term nearly cancels the code term (dmin*mn within a few percent of d*sc*q for the
    # codes present): sum |x*w| is far smaller than B. The M <= 2 bound is stated against B and must hold.
    rng = np.random.Generator(np.random.PCG64(4500 + M))
    N, K = 64, 2048
    blocks = synth.random_blocks(rng, N * K // QK_K).reshape(N * K // QK_K, BB).copy()
    blocks[:, 16:80] = 0xAA                                             # every code 2
    sc = rng.integers(1, 16, (blocks.shape[0], 16))
    blocks[:, 0:16] = (sc | (sc << 4)).astype(np.uint8)                 # mn = sc
    d = rng.uniform(0.05, 0.2, blocks.shape[0]).astype(np.float16)
    dmin = (d.astype(np.float64) * 2 * (1 + rng.uniform(-0.03, 0.03, blocks.shape[0]))).astype(np.float16)
    blocks[:, 80:82] = d.view(np.uint8).reshape(-1, 2)
    blocks[:, 82:84] = dmin.view(np.uint8).reshape(-1, 2)
    blocks = blocks.reshape(-1)
    x = rng.standard_normal((M, K), dtype=np.float32)
    y = gpu_matmul(x, blocks, M, N, K)
    ref, a = oracle.matmul(x, blocks, M, N, K)
    b = _b_bound(x, blocks, M, N, K)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= _m2_bound(K) * b)
    print("near cancellation, M=%d: B/A up to %.3g, max err/B = %.3g, max err/A = %.3g" % (
        M, np.max(b / a), np.max(err / b), np.max(err / a)))


@pytest.mark.parametrize("M", [3, 8])
def test_gemv_matrix_cores_meet_the_fp32_rule_within_a_2_pow_10_spread(M):
    # 3 <= M <= 8: the matrix cores sum the 32 exact products of a step within a window of about 2^16 below its
    # largest; codes span up to 45 (2^5.5), so activations spanning up to 2^10 inside a 256-weight block keep
    # every product in the window and the 1e-5 rule holds. Here every block row spans the full 2^10.
    rng = np.random.Generator(np.random.PCG64(4600 + M))
    N, K = 300, 4096
    blocks = synth.random_blocks(rng, N * K // QK_K)
    mag = 2.0 ** rng.uniform(-10, 0, (M, K))
    mag[:, ::256] = 1.0                                                 # each block row reaches its top
    x = (mag * rng.choice([-1.0, 1.0], (M, K))).astype(np.float32)
    y = gpu_matmul(x, blocks, M, N, K)
    worst = check_gemv(y, x, blocks, M, N, K)
    print("matrix-core GEMV, activations spanning 2^10 per block, M=%d: max err/A = %.3g" % (M, worst))


@pytest.mark.parametrize("M", [3, 8])
def test_gemv_matrix_cores_beyond_the_window_lose_only_small_products(M):
    # The case the fp32 rule does not cover for 3 <= M <= 8: each block row's largest activation sits on a zero
    # weight and the others are 1e-7 of it, so the activations that count are split into f16 pieces far below
    # the block's scale. The stated bound is relative to the block maxima:
    #   |y - exact| <= 2^-18 B + 2^-6 sum_b max_k|x| (max_k |d*sc*q| + 16 max_s |dmin*mn|).
    rng = np.random.Generator(np.random.PCG64(4700 + M))
    N, K = 64, 1024
    blocks = synth.random_blocks(rng, N * K // QK_K).reshape(N, K // QK_K, BB).copy()
    blocks[:, :, 16] &= 0xFC                                            # element 0 of each block: code 0
    blocks[:, :, 0] &= 0x0F                                             # and min nibble 0: weight exactly 0
    blocks = blocks.reshape(-1)
    assert np.all(oracle.dequantize(blocks).reshape(N, K)[:, ::256] == 0.0)
    x = (rng.standard_normal((M, K)) * 1e-7).astype(np.float32)
    x[:, ::256] = 1.0
    y = gpu_matmul(x, blocks, M, N, K)
    ref, a = oracle.matmul(x, blocks, M, N, K)
    bound = _m8_bound(x, blocks, M, N, K)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= bound)
    print("matrix-core GEMV, block maxima on zero weights, M=%d: max err/A = %.3g, max err/bound = %.3g" % (
        M, np.max(err / a), np.max(err / bound)))
