"""GPU argmax / threshold-candidate collect against the oracle, bit for bit.

Operation: docs.rs source page of mlx-native 0.9.5, src/mlx_native/ops/gpu_sample.rs
(first-max argmax with lower-index tie-break, candidates are logits >=
top1 - 0.5f, the count may exceed cap, overflow flag). Every output is
integer or a copied logit, so parity is exact: indices, the top1 value's bits,
counts, flags and the first min(count, cap) candidate ids in increasing order.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
import ggml_q2_dequant_amd as q2k  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q2k.load_library()
    yield
    torch.cuda.synchronize()


def run(x, n_slots, vocab, cap):
    d = "cuda:0"
    lg = torch.from_numpy(np.ascontiguousarray(x, np.float32).reshape(n_slots, vocab)).to(d)
    idx = torch.full((n_slots,), 0xABCD, dtype=torch.int32, device=d)
    val = torch.full((n_slots,), -7.0, dtype=torch.float32, device=d)
    cnt = torch.full((n_slots,), -1, dtype=torch.int32, device=d)
    ovf = torch.full((n_slots,), -1, dtype=torch.int32, device=d)
    ids = torch.full((n_slots, cap), -1, dtype=torch.int32, device=d)
    q2k.q2k_argmax_candidates(lg, n_slots, vocab, cap, idx, val, cnt, ovf, ids)
    torch.cuda.synchronize()
    return (idx.cpu().numpy().view(np.uint32), val.cpu().numpy(), cnt.cpu().numpy().view(np.uint32),
            ovf.cpu().numpy().view(np.uint32), ids.cpu().numpy().view(np.uint32))


def check(x, n_slots, vocab, cap):
    gi, gv, gc, go, gids = run(x, n_slots, vocab, cap)
    ri, rv, rc, ro, rids = oracle.argmax_candidates(x, n_slots, vocab, cap)
    assert np.array_equal(gi, ri)
    assert np.array_equal(gv.view(np.uint32), rv.view(np.uint32))
    assert np.array_equal(gc, rc) and np.array_equal(go, ro)
    for s in range(n_slots):
        n = min(int(rc[s]), cap)
        assert np.array_equal(gids[s, :n], rids[s])
        assert np.all(gids[s, n:] == 0xFFFFFFFF)  # entries past the candidates are left unwritten
    return gi, gc


def test_page_scale_vocab_with_planted_candidates():
    # vocab 262144 as in the page's decode context; a few logits planted just
    # under the maximum, some exactly on the threshold.
    rng = np.random.Generator(np.random.PCG64(71))
    n_slots, vocab, cap = 5, 262144, 32
    x = rng.standard_normal((n_slots, vocab)).astype(np.float32)
    for s in range(n_slots):
        top = np.float32(9.0 + s)
        pos = rng.choice(vocab, 12, replace=False)
        x[s, pos[0]] = top
        x[s, pos[1:6]] = top - np.float32(0.5)          # exactly on the threshold: included
        x[s, pos[6:9]] = np.nextafter(top - np.float32(0.5), np.float32(-np.inf))  # just below
        x[s, pos[9:]] = top - np.float32(0.25)
    gi, gc = check(x, n_slots, vocab, cap)
    assert np.all(gc == 9)


# Chunks are 4096 logits up to a 2^18 vocabulary (one round of 16 steps per wavefront), longer beyond
# it (rounds of 32 steps, the last one partial).
@pytest.mark.parametrize("n_slots,vocab,cap", [(1, 1, 1), (3, 7, 2), (2, 300, 512), (4, 4096, 5), (2, 4097, 64),
                                               (4, 8192, 5), (2, 8193, 64), (3, 65537, 9), (2, 262145, 33),
                                               (1, 600001, 100)])
def test_ragged_sizes_and_chunk_edges(n_slots, vocab, cap):
    rng = np.random.Generator(np.random.PCG64(n_slots * 7 + vocab))
    x = (rng.integers(0, 6, (n_slots, vocab)).astype(np.float32) * np.float32(0.25))  # many ties and candidates
    check(x, n_slots, vocab, cap)


def test_ties_across_chunks_take_the_lowest_index():
    vocab = 3 * 8192 + 17
    x = np.zeros((3, vocab), np.float32)
    x[0, [9000, 20000, vocab - 1]] = 1.0
    x[1, [vocab - 1, 5]] = 1.0
    x[2, [4096, 4095 + 4096, 4095]] = 1.0  # first and last column of neighbouring 4096-logit chunks
    gi, _ = check(x, 3, vocab, 4)
    assert gi.tolist() == [9000, 5, 4095]


def test_nan_and_infinity_rows():
    vocab = 20000
    x = np.ones((4, vocab), np.float32)
    x[0, 0] = np.nan                       # NaN in column 0: the answer, no candidates
    x[1, 100:200] = np.nan
    x[1, 15000] = 4.0                      # NaN elsewhere is passed over
    x[2, :] = -np.inf                      # all -inf: every column is a candidate
    x[3, 123] = np.inf
    x[3, 19999] = np.inf
    check(x, 4, vocab, 16)


def test_overflow_flag_and_capacity():
    x = np.zeros((3, 10000), np.float32)
    x[1, ::2] = -1.0
    check(x, 3, 10000, 7)


def test_more_slots_than_one_launch_covers():
    rng = np.random.Generator(np.random.PCG64(72))
    n_slots, vocab, cap = 65537, 3, 2
    x = rng.integers(0, 3, (n_slots, vocab)).astype(np.float32)
    check(x, n_slots, vocab, cap)
