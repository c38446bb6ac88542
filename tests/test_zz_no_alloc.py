"""q2k_matmul_noalloc, the matmul entry point that allocates nothing, through the C ABI.

Its output must equal q2k_matmul's bit for bit (the same kernels; only where
bf16(x) is staged differs: the library's file-scope device array instead of the
per-stream workspace), and q2k_matmul's result is in turn held to the oracle's
rule for its path. Two calls in a row, the second smaller, show that a call
does not depend on what the previous one left in the shared array. Sizes whose
bf16 activations exceed the array are rejected before anything is enqueued.
The call is meant for code under HIP graph capture: a captured call replays
correctly with new activations, with eager calls of its own (which overwrite the
shared array) between the replays.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import ggml_q2_dequant_amd as q2k  # noqa: E402

pytestmark = pytest.mark.gpu

QK_K = 256


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return q2k.load_library()


def _run(lib, fn, x, w, M, N, K):
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    rc = getattr(lib, fn)(x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, K,
                          torch.cuda.current_stream().cuda_stream)
    assert rc == q2k.Q2K_OK, lib.q2k_last_error_message().decode()
    return y


def _problem(seed, M, N, K):
    rng = np.random.Generator(np.random.PCG64(seed))
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    return x, blocks, torch.from_numpy(x).to("cuda:0"), torch.from_numpy(blocks).to("cuda:0")


def test_noalloc_matches_matmul_on_two_calls_the_second_smaller(lib):
    results = []
    for seed, (M, N, K) in ((8100, (512, 1000, 4096)), (8101, (40, 300, 768))):
        print("noalloc call M=%d N=%d K=%d" % (M, N, K), flush=True)
        x_h, w_h, x, w = _problem(seed, M, N, K)
        y_na = _run(lib, "q2k_matmul_noalloc", x, w, M, N, K)
        torch.cuda.synchronize()
        y_ref = _run(lib, "q2k_matmul", x, w, M, N, K)
        torch.cuda.synchronize()
        a, b = y_na.cpu().numpy(), y_ref.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        ref, amag = oracle.matmul(x_h, w_h, M, N, K, nthreads=oracle.host_threads())
        assert np.all(np.abs(a.astype(np.float64) - ref) <= 4e-3 * amag + 1e-6)
        results.append(a)
    assert results[1].shape == (40, 300)


def test_noalloc_small_m_uses_the_gemv_and_needs_no_scratch(lib):
    x_h, w_h, x, w = _problem(8102, 3, 257, 1280)
    y_na = _run(lib, "q2k_matmul_noalloc", x, w, 3, 257, 1280)
    y_ref = _run(lib, "q2k_matmul", x, w, 3, 257, 1280)
    torch.cuda.synchronize()
    assert np.array_equal(y_na.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32))
    ref, amag = oracle.matmul(x_h, w_h, 3, 257, 1280)
    assert np.all(np.abs(y_na.cpu().numpy().astype(np.float64) - ref) <= 1e-5 * amag)


def test_noalloc_rejects_activations_larger_than_its_array(lib):
    # 2 * M * K must stay within 16 MiB: M = 2049, K = 4096 needs 16 MiB + 8 KiB. Validation only: the
    # pointers are never dereferenced because the call fails before enqueuing anything.
    M, N, K = 2049, 16, 4096
    y = torch.zeros(64, dtype=torch.float32, device="cuda:0")
    rc = lib.q2k_matmul_noalloc(1 << 32, 2 << 32, y.data_ptr(), M, N, K, None)
    assert rc == q2k.Q2K_ERR_INVALID_ARGUMENT
    assert "device scratch holds" in lib.q2k_last_error_message().decode()
    x = torch.zeros(2048 * 4096, dtype=torch.float32, device="cuda:0")
    w = torch.zeros(16 * 16 * 84, dtype=torch.uint8, device="cuda:0")
    yy = _run(lib, "q2k_matmul_noalloc", x, w, 2048, 16, 4096)   # exactly 16 MiB: accepted
    torch.cuda.synchronize()
    assert torch.all(yy == 0)
    assert ctypes.sizeof(ctypes.c_void_p) == 8


def test_noalloc_call_captured_in_a_graph_replays_with_new_activations(lib):
    # Capture one M=200 matrix-core call (its bf16 staging in the library's array), then replay it three
    # times; before each replay the activations change and an eager call of another shape overwrites the
    # array. Every replay must equal q2k_matmul on the same activations, bit for bit.
    M, N, K = 200, 384, 1024
    rng = np.random.Generator(np.random.PCG64(8103))
    w_h = synth.random_blocks(rng, N * K // QK_K)
    xs_h = [rng.standard_normal((M, K), dtype=np.float32) for _ in range(4)]
    w = torch.from_numpy(w_h).to("cuda:0")
    x = torch.from_numpy(xs_h[0]).to("cuda:0")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    x_o, w_o = torch.from_numpy(rng.standard_normal((64, 512), dtype=np.float32)).to("cuda:0"), \
        torch.from_numpy(synth.random_blocks(rng, 96 * 512 // QK_K)).to("cuda:0")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        _run(lib, "q2k_matmul_noalloc", x, w, M, N, K)       # the array's address is looked up eagerly
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            rc = lib.q2k_matmul_noalloc(x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, K,
                                        torch.cuda.current_stream().cuda_stream)
        assert rc == q2k.Q2K_OK, lib.q2k_last_error_message().decode()
        torch.cuda.synchronize()
        for r in range(1, 4):
            print("noalloc graph replay %d" % r, flush=True)
            x.copy_(torch.from_numpy(xs_h[r]).to("cuda:0"))
            _run(lib, "q2k_matmul_noalloc", x_o, w_o, 64, 96, 512)   # eager work on the shared array
            torch.cuda.synchronize()
            y.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            want = _run(lib, "q2k_matmul", x, w, M, N, K)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint32), want.cpu().numpy().view(np.uint32)), r
    del g
