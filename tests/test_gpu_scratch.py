"""GPU tests of device scratch: the caller-held (pooled) forms and the library's per-stream workspace.

* q2k_matmul_pooled and q2k_argmax_candidates_pooled give, bit for bit, what the
  workspace forms give (the same kernels on the same inputs), and the oracle's
  answer within the path's rule.
* The per-stream workspace only grows and never frees a buffer a graph may hold:
  a graph captured with an M > 8 call still replays correctly after an eager call
  with a larger M on the same stream (the buffer it captured was retired, not freed).
* Growth during capture is refused with an error and enqueues nothing.
* The synchronous gather (it waits on the host) is refused during capture; the
  asynchronous gather captures and replays.
The page behind the pooled forms is the docs.rs source page of mlx-native 0.10.8,
tests/deepseek_q2_k.rs (caller-held IdMmScratch for the pooled expert-routed calls)
and the op helpers of mlx-native 0.21.1, src/ops/dflash2_selector.rs (caller-owned,
reusable workspace buffers, no allocation in the call).
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import ggml_q2_dequant_amd as q2k  # noqa: E402

pytestmark = pytest.mark.gpu

QK_K = 256


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q2k.load_library()
    yield
    torch.cuda.synchronize()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _problem(seed, M, N, K):
    rng = np.random.Generator(np.random.PCG64(seed))
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    return x, blocks


@pytest.mark.parametrize("M,N,K,path", [(40, 300, 768, q2k.PATH_AUTO), (3, 70, 512, q2k.PATH_AUTO),
                                        (1, 33, 256, q2k.PATH_MFMA), (130, 257, 1280, q2k.PATH_MFMA)])
def test_matmul_pooled_equals_workspace_form(M, N, K, path):
    x_h, w_h = _problem(7000 + M + N, M, N, K)
    x, w = dev(x_h), dev(w_h)
    need = q2k.q2k_matmul_scratch_bytes(M, N, K, path)
    resolved_mfma = path == q2k.PATH_MFMA or (path == q2k.PATH_AUTO and M > 8)
    assert need == (2 * M * K if resolved_mfma else 0)
    scratch = torch.full((max(need, 1) // 4 + 64,), -1, dtype=torch.int32, device="cuda:0") if need else None
    y1 = torch.full((M, N), float("nan"), device="cuda:0")
    y2 = torch.full((M, N), float("nan"), device="cuda:0")
    q2k.q2k_matmul_path(x, w, y1, M, N, K, path)
    q2k.q2k_matmul_pooled(x, w, y2, M, N, K, scratch, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y1), bits(y2))
    ref, a = oracle.matmul(x_h, w_h, M, N, K)
    err = np.abs(y2.cpu().numpy().astype(np.float64) - ref)
    if resolved_mfma:
        assert np.all(err <= 4e-3 * a + 1e-6)
    else:
        assert np.all(err <= 1e-5 * a)


def test_argmax_pooled_equals_workspace_form():
    ns, vocab, cap = 3, 70001, 16
    rng = np.random.Generator(np.random.PCG64(7100))
    lg_h = rng.standard_normal((ns, vocab), dtype=np.float32)
    lg_h[1, [5, 60000]] = 9.0
    lg = dev(lg_h)
    outs = [[torch.full((ns,), -1, dtype=torch.int32, device="cuda:0") for _ in range(4)] +
            [torch.full((ns, cap), -1, dtype=torch.int32, device="cuda:0")] for _ in range(2)]
    q2k.q2k_argmax_candidates(lg, ns, vocab, cap, outs[0][0], outs[0][1], outs[0][2], outs[0][3], outs[0][4])
    need = q2k.q2k_argmax_candidates_scratch_bytes(ns, vocab)
    scratch = torch.empty((need + 255) // 4 + 64, dtype=torch.int32, device="cuda:0")
    q2k.q2k_argmax_candidates_pooled(lg, ns, vocab, cap, outs[1][0], outs[1][1], outs[1][2], outs[1][3], outs[1][4],
                                     scratch)
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(bits(a), bits(b))
    idx, val, cnt, ovf, ids = oracle.argmax_candidates(lg_h, ns, vocab, cap)
    got_idx = outs[1][0].cpu().numpy().view(np.uint32)
    assert np.array_equal(got_idx, idx)
    for s in range(ns):
        c = int(outs[1][2][s].item())
        assert c == int(cnt[s])
        assert np.array_equal(outs[1][4][s, :min(c, cap)].cpu().numpy().view(np.uint32), ids[s])


def test_graph_replay_after_a_larger_eager_call_on_the_capture_stream():
    # Capture an M=200 matrix-core call, then make an eager M=1024 call on the same
    # stream (the workspace grows; the captured buffer is retired, not freed), then
    # replay the graph several times with eager work between: every replay must equal
    # the eager M=200 result.
    N, K = 384, 1024
    x_big_h, w_h = _problem(7200, 1024, N, K)
    w = dev(w_h)
    x_small, x_big = dev(x_big_h[:200].copy()), dev(x_big_h)
    y_small_eager = torch.full((200, N), float("nan"), device="cuda:0")
    y_big = torch.full((1024, N), float("nan"), device="cuda:0")
    y_graph = torch.full((200, N), float("nan"), device="cuda:0")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        q2k.q2k_matmul(x_small, w, y_small_eager, 200, N, K)   # sizes the workspace outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            q2k.q2k_matmul(x_small, w, y_graph, 200, N, K)
        torch.cuda.synchronize()
        q2k.q2k_matmul(x_big, w, y_big, 1024, N, K)              # grows the stream's workspace
        torch.cuda.synchronize()
        for r in range(3):
            y_graph.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits(y_graph), bits(y_small_eager)), "replay %d differs" % r
            q2k.q2k_matmul(x_big, w, y_big, 1024, N, K)          # eager work on the stream between replays
            torch.cuda.synchronize()
    assert np.array_equal(bits(y_big[:200]), bits(y_small_eager))  # rows do not depend on M's other rows' count
    del g


def test_workspace_growth_is_refused_during_capture():
    N, K, M = 64, 512, 4096
    x_h, w_h = _problem(7300, M, N, K)
    x, w = dev(x_h), dev(w_h)
    y = torch.zeros((M, N), device="cuda:0")
    s = torch.cuda.Stream()   # a new stream: its workspace is empty
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with pytest.raises(q2k.Q2KInvalidArgument, match="graph capture"):
            with torch.cuda.graph(g, stream=s):
                y.fill_(1.0)
                q2k.q2k_matmul(x, w, y, M, N, K)
        torch.cuda.synchronize()
        # The same call made eagerly first, then captured, works.
        q2k.q2k_matmul(x, w, y, M, N, K)
        torch.cuda.synchronize()
        want = y.clone()
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=s):
            q2k.q2k_matmul(x, w, y, M, N, K)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), want.view(torch.int32))
    del g, g2


def test_synchronous_gather_is_refused_during_capture_and_the_asynchronous_one_replays():
    # The synchronous gather waits on the host for its kernel, which a capture
    # cannot hold: it must be refused before anything is enqueued. The
    # asynchronous form captures; every replay must match the eager result.
    vocab, dim = 3, QK_K
    table_h = np.concatenate([synth.page_block(r + 2) for r in range(vocab)])
    table, ids = dev(table_h), dev(np.array([2, 0, 1, 2], dtype=np.uint32))
    want = oracle.gather(table_h, [2, 0, 1, 2], vocab, dim, 4)
    out = torch.full((4, dim), float("nan"), device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with pytest.raises(q2k.Q2KInvalidArgument, match="cannot be captured"):
            with torch.cuda.graph(g, stream=s):
                out.fill_(0.0)   # something captured besides the refused call
                q2k.q2k_embedding_gather(table, ids, out, vocab, dim, 4, stream=s)
        torch.cuda.synchronize()
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=s):
            q2k.q2k_embedding_gather_async(table, ids, out, vocab, dim, 4, status, stream=s)
        for r in range(3):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g2.replay()
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32)), "replay %d differs" % r
            assert int(status.item()) == 0
            q2k.q2k_embedding_gather(table, ids, out, vocab, dim, 4, stream=s)   # eager work between replays
            torch.cuda.synchronize()
    del g, g2
