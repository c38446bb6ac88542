"""GPU parity of the expert-routed product (q2k_matmul_id family) against the oracle.

The page is the docs.rs source page of mlx-native 0.10.8, tests/deepseek_q2_k.rs:
fn run_expert (its tests q2_k_expert_routed_metal_matches_reference = (2, 2, 3),
q2_k_expert_mm_id_top_k_6_matches_reference = (33, 6, 8) through the pooled pair,
q2_k_public_prefill_top_k_6_matches_reference = (33, 6, 8) through the plain call)
and test q2_k_slotted_down_mm_is_byte_identical_to_flattened_rows.

Rules: the fp32 per-route schedule meets |y - exact| <= 1e-5 * sum|x*w| (and the
page's 2e-4 on its fixtures) and each route's row is bit-identical to q2k_matmul
with M = 1 on that expert; the matrix-core schedule meets the bf16 rules of the
dense path (4e-3 * sum|x*w| + 1e-6, and the fp32-accumulation bound against the
oracle on bf16-rounded operands), and each expert's rows are bit-identical to the
dense matrix-core product of that expert with its routed rows in route order.
Byte-identities: pair outputs with equal weights, slotted = flattened, pooled =
workspace call. Routes with an id >= n_experts give NaN rows and raise the status
word. Inputs: the page fixtures and seeded random routings (synth).
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
    yield
    torch.cuda.synchronize()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def params(tokens, top_k, n, K, experts, stride=None):
    return q2k.MatmulIdParams(n_tokens=tokens, top_k=top_k, n=n, k=K, n_experts=experts, reserved=0,
                              expert_stride=stride if stride is not None else n * (K // QK_K) * BB)


def bits_equal(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return a.shape == b.shape and np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32),
                                                                            b[~nb].view(np.uint32))


class Run:
    """Device copies of one problem and the calls that fill fresh outputs."""

    def __init__(self, x, w, ids, p, slotted=False):
        self.p, self.slotted = p, slotted
        self.routes = p.n_tokens * p.top_k
        self.xd, self.wd, self.idd = dev(x.astype(np.float32)), dev(w), dev(np.asarray(ids, np.uint32))
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def out(self):
        return torch.full((self.routes, self.p.n), 7.0, dtype=torch.float32, device="cuda:0")

    def scratch(self):
        nb = q2k.q2k_matmul_id_scratch_bytes(self.p)
        assert nb > 0
        # Garbage contents: the call must not depend on them.
        return torch.randint(0, 255, (nb,), dtype=torch.uint8, device="cuda:0")

    def plain(self, path=q2k.PATH_AUTO):
        assert not self.slotted
        y = self.out()
        q2k.q2k_matmul_id_path(self.xd, self.wd, self.idd, y, self.p, path, status=self.status)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def pooled(self):
        y = self.out()
        call = q2k.q2k_matmul_id_pooled_slotted if self.slotted else q2k.q2k_matmul_id_pooled
        call(self.xd, self.wd, self.idd, y, self.p, self.scratch(), status=self.status)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def pair(self, w1):
        y0, y1 = self.out(), self.out()
        q2k.q2k_matmul_id_pooled_pair(self.xd, self.wd, dev(w1), self.idd, y0, y1, self.p, self.scratch(),
                                      status=self.status)
        torch.cuda.synchronize()
        return y0.cpu().numpy(), y1.cpu().numpy()

    def flagged(self):
        return int(self.status.cpu().item())


def oracle_id(x, w, ids, p, slotted=False, bf16=False):
    return oracle.matmul_id(x, w, ids, p.n_tokens, p.top_k, p.n, p.k, p.n_experts, p.expert_stride,
                            slotted=slotted, bf16_operands=bf16, nthreads=oracle.host_threads())


def check_gemv(y, x, w, ids, p, slotted=False):
    ref, a, bad = oracle_id(x, w, ids, p, slotted)
    nan_rows = np.isnan(ref[:, 0])
    assert np.all(np.isnan(y[nan_rows]))
    yv, rv, av = y[~nan_rows].astype(np.float64), ref[~nan_rows], a[~nan_rows]
    assert np.all(np.isfinite(yv))
    err = np.abs(yv - rv)
    assert np.all(err <= GEMV_REL * av), "max |err|/A = %g" % float(np.max(err / av))
    return ref, bad


def check_mfma(y, x, w, ids, p, slotted=False):
    ref, a, bad = oracle_id(x, w, ids, p, slotted)
    refb, ab, _ = oracle_id(x, w, ids, p, slotted, bf16=True)
    nan_rows = np.isnan(ref[:, 0])
    assert np.all(np.isnan(y[nan_rows]))
    yv = y[~nan_rows].astype(np.float64)
    assert np.all(np.isfinite(yv))
    err = np.abs(yv - ref[~nan_rows])
    assert np.all(err <= MFMA_REL * a[~nan_rows] + MFMA_ABS), "max |err|/A = %g" % float(np.max(err / a[~nan_rows]))
    errb = np.abs(yv - refb[~nan_rows])
    assert np.all(errb <= p.k * 2.0 ** -24 * ab[~nan_rows] + MFMA_ABS)
    return ref, bad


def expert_rows(w, p, e):
    stride = p.expert_stride
    return w[e * stride:e * stride + p.n * (p.k // QK_K) * BB]


def dense(xrows, wrows, N, K, path):
    xd, wd = dev(np.ascontiguousarray(xrows, np.float32)), dev(wrows)
    y = torch.empty((xrows.shape[0], N), dtype=torch.float32, device="cuda:0")
    q2k.q2k_matmul_path(xd, wd, y, xrows.shape[0], N, K, path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_routes_match_dense(y, x, w, ids, p, path, slotted=False):
    """Each expert's rows equal the dense product of that expert with its routed rows in route order."""
    ids = np.asarray(ids)
    for e in range(p.n_experts):
        routes = np.nonzero(ids == e)[0]
        if routes.size == 0:
            continue
        xrows = x[routes] if slotted else x[routes // p.top_k]
        if path == q2k.PATH_GEMV:  # one M = 1 call per route
            for r, xr in zip(routes, xrows):
                assert bits_equal(y[r], dense(xr[None, :], expert_rows(w, p, e), p.n, p.k, path)[0])
        else:
            assert bits_equal(y[routes], dense(xrows, expert_rows(w, p, e), p.n, p.k, path))


# ----------------------------------------------------------------- the page's tests

def _page(tokens, top_k, experts, n=8):
    w = synth.page_expert_weights(experts, n)
    x = synth.page_input(tokens).reshape(tokens, QK_K)
    return x, w, synth.page_routes(tokens, top_k, experts), params(tokens, top_k, n, QK_K, experts)


def test_page_expert_routed_2_2_3_uses_fp32_and_meets_2e4():
    x, w, ids, p = _page(2, 2, 3)
    run = Run(x, w, ids, p)
    y = run.plain()
    ref, bad = check_gemv(y, x, w, ids, p)
    assert bad == 0 and run.flagged() == 0
    assert np.all(np.abs(y - ref) <= 2e-4)
    assert bits_equal(y, run.plain(q2k.PATH_GEMV))  # AUTO picks the fp32 schedule here
    check_routes_match_dense(y, x, w, ids, p, q2k.PATH_GEMV)


def test_page_public_prefill_33_6_8_uses_matrix_cores():
    x, w, ids, p = _page(33, 6, 8)
    run = Run(x, w, ids, p)
    y = run.plain()
    check_mfma(y, x, w, ids, p)
    assert bits_equal(y, run.plain(q2k.PATH_MFMA))
    assert run.flagged() == 0
    check_routes_match_dense(y, x, w, ids, p, q2k.PATH_MFMA)


def test_page_mm_id_pair_33_6_8_prepared_equals_ordinary():
    x, w, ids, p = _page(33, 6, 8)
    run = Run(x, w, ids, p)
    y0, y1 = run.pair(w)
    assert bits_equal(y0, y1)
    check_mfma(y0, x, w, ids, p)
    assert bits_equal(y0, run.pooled())
    assert bits_equal(y0, run.plain(q2k.PATH_MFMA))


def test_page_slotted_down_is_byte_identical_to_flattened():
    tokens, top_k, experts, n = 33, 6, 8, 8
    w = synth.page_expert_weights(experts, n)
    xr = synth.page_input(tokens * top_k).reshape(tokens * top_k, QK_K)
    ids = synth.page_routes(tokens, top_k, experts)
    flat = Run(xr, w, ids, params(tokens * top_k, 1, n, QK_K, experts))
    slot = Run(xr, w, ids, params(tokens, top_k, n, QK_K, experts), slotted=True)
    yf, ys = flat.pooled(), slot.pooled()
    assert bits_equal(yf, ys)
    check_mfma(ys, xr, w, ids, slot.p, slotted=True)


# ----------------------------------------------------------------- seeded routings

def _random(seed, tokens, top_k, experts, n, K, skew=False, stride_pad=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    rb = (K // QK_K) * BB
    blocks = synth.random_blocks(rng, experts * n * K // QK_K)
    if stride_pad:
        w = np.full(experts * (n * rb + stride_pad), 0xFF, dtype=np.uint8)  # 0xFFFF d: NaN if ever read
        for e in range(experts):
            w[e * (n * rb + stride_pad):e * (n * rb + stride_pad) + n * rb] = blocks[e * n * rb:(e + 1) * n * rb]
    else:
        w = blocks
    x = rng.standard_normal((tokens, K)).astype(np.float32)
    if skew:  # most routes on expert 0, several experts empty
        ids = np.where(rng.random(tokens * top_k) < 0.7, 0, rng.integers(0, max(experts // 3, 1), tokens * top_k))
        ids = ids.astype(np.uint32)
    else:
        ids = synth.random_routes(rng, tokens, top_k, experts)
    return x, w, ids, params(tokens, top_k, n, K, experts, n * rb + stride_pad)


CASES = {
    # name: (seed, tokens, top_k, experts, n, K, skew, pad)
    "two_tiles_per_expert_ragged_n": (71, 300, 2, 4, 520, 512, False, 0),
    "top8_of_16_many_small_groups": (72, 40, 8, 16, 264, 768, False, 0),
    "skewed_with_empty_experts": (73, 180, 3, 12, 256, 256, True, 0),
    "padded_expert_stride": (74, 50, 6, 8, 130, 1024, False, 3 * BB + 4),
    "top_k_above_experts_duplicates": (75, 20, 5, 3, 72, 256, False, 0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_matrix_core_schedule_on_seeded_routings(name):
    seed, tokens, top_k, experts, n, K, skew, pad = CASES[name]
    print("moe mfma case", name, flush=True)
    x, w, ids, p = _random(seed, tokens, top_k, experts, n, K, skew, pad)
    run = Run(x, w, ids, p)
    y = run.plain(q2k.PATH_MFMA)
    check_mfma(y, x, w, ids, p)
    assert run.flagged() == 0
    assert bits_equal(y, run.pooled())
    check_routes_match_dense(y, x, w, ids, p, q2k.PATH_MFMA)


@pytest.mark.parametrize("name", sorted(CASES))
def test_fp32_schedule_on_seeded_routings(name):
    seed, tokens, top_k, experts, n, K, skew, pad = CASES[name]
    print("moe gemv case", name, flush=True)
    x, w, ids, p = _random(seed, min(tokens, 24), top_k, experts, n, K, skew, pad)
    run = Run(x, w, ids, p)
    y = run.plain(q2k.PATH_GEMV)
    check_gemv(y, x, w, ids, p)
    assert run.flagged() == 0
    check_routes_match_dense(y, x, w, ids, p, q2k.PATH_GEMV)


@pytest.mark.parametrize("path", [q2k.PATH_GEMV, q2k.PATH_MFMA])
def test_bad_ids_give_nan_rows_and_raise_status(path):
    x, w, ids, p = _random(76, 40, 6, 8, 96, 512)
    ids = ids.copy()
    ids[[3, 100, 239]] = [8, 0xFFFFFFFF, 1000]
    run = Run(x, w, ids, p)
    y = run.plain(path)
    assert run.flagged() == 1
    (check_gemv if path == q2k.PATH_GEMV else check_mfma)(y, x, w, ids, p)
    assert np.all(np.isnan(y[[3, 100, 239]]))
    good = np.ones(p.n_tokens * p.top_k, bool)
    good[[3, 100, 239]] = False
    assert np.all(np.isfinite(y[good]))


def test_pair_with_different_weights_equals_two_pooled_calls():
    x, w0, ids, p = _random(77, 64, 6, 8, 200, 512)
    _, w1, _, _ = _random(78, 64, 6, 8, 200, 512)
    y0, y1 = Run(x, w0, ids, p).pair(w1)
    assert bits_equal(y0, Run(x, w0, ids, p).pooled())
    assert bits_equal(y1, Run(x, w1, ids, p).pooled())
    check_mfma(y1, x, w1, ids, p)


def test_slotted_on_seeded_routing_equals_flattened_and_oracle():
    tokens, top_k, experts, n, K = 45, 6, 8, 136, 768
    x, w, ids, _ = _random(79, tokens * top_k, 1, experts, n, K)
    ids = synth.random_routes(np.random.Generator(np.random.PCG64(80)), tokens, top_k, experts)
    slot = Run(x, w, ids, params(tokens, top_k, n, K, experts), slotted=True)
    flat = Run(x, w, ids, params(tokens * top_k, 1, n, K, experts))
    ys = slot.pooled()
    assert bits_equal(ys, flat.pooled())
    check_mfma(ys, x, w, ids, slot.p, slotted=True)


def test_matrix_core_tiles_with_exact_multiples_and_partial_only_experts():
    # Expert 0 fills exactly two 128-row tiles, expert 1 is empty, experts 2
    # and 3 have only partial tiles: the tile list holds the full tiles first
    # and the partial ones after them.
    tokens, top_k, experts, n, K = 200, 2, 4, 136, 512
    rng = np.random.Generator(np.random.PCG64(91))
    rb = (K // QK_K) * BB
    w = synth.random_blocks(rng, experts * n * K // QK_K)
    x = rng.standard_normal((tokens, K)).astype(np.float32)
    ids = np.array([0] * 256 + [2] * 100 + [3] * 44, dtype=np.uint32)
    rng.shuffle(ids)
    p = params(tokens, top_k, n, K, experts, n * rb)
    run = Run(x, w, ids, p)
    y = run.plain(q2k.PATH_MFMA)
    check_mfma(y, x, w, ids, p)
    assert run.flagged() == 0
    assert bits_equal(y, run.pooled())
    check_routes_match_dense(y, x, w, ids, p, q2k.PATH_MFMA)


def test_single_token_and_single_expert_edges():
    for tokens, top_k, experts in ((1, 1, 1), (1, 6, 8), (33, 1, 1)):
        x, w, ids, p = _random(81 + tokens + top_k, tokens, top_k, experts, 40, 256)
        run = Run(x, w, ids, p)
        check_gemv(run.plain(q2k.PATH_GEMV), x, w, ids, p)
        check_mfma(run.plain(q2k.PATH_MFMA), x, w, ids, p)


# ----------------------------------------------------------------- full-size workloads, every output

def _check_every_route(y, inp, bf16):
    """Every route of a full-size workload against the oracle. A route's row is the dense product of its
    activation row with its expert's weights (fn run_expert), so the oracle runs once per expert on the
    rows routed to it, which decodes each weight row once instead of once per route."""
    import time
    c = inp.config
    rb = (c.K // QK_K) * BB
    t0 = time.perf_counter()
    worst = 0.0
    first_expert = int(inp.ids[0])
    for e in range(c.experts):
        routes = np.nonzero(inp.ids == e)[0]
        if routes.size == 0:
            continue
        xs = np.ascontiguousarray(inp.x[routes // c.top_k])
        we = inp.blocks[e * c.n * rb:(e + 1) * c.n * rb]
        ref, a = oracle.matmul(xs, we, routes.size, c.n, c.K, nthreads=oracle.host_threads())
        ye = y[routes].astype(np.float64)
        err = np.abs(ye - ref)
        if bf16:
            assert np.all(err <= MFMA_REL * a + MFMA_ABS), "expert %d: max |err|/A = %g" % (e, np.max(err / a))
            if e == first_expert:
                # The tighter bound against the oracle on bf16-rounded operands, on one expert's routes
                # (that oracle pass costs about three times the f64 one).
                refb, ab = oracle.matmul(xs, we, routes.size, c.n, c.K, bf16_operands=True,
                                         nthreads=oracle.host_threads())
                assert np.all(np.abs(ye - refb) <= c.K * 2.0 ** -24 * ab + MFMA_ABS)
        else:
            assert np.all(err <= GEMV_REL * a), "expert %d: max |err|/A = %g" % (e, np.max(err / a))
        worst = max(worst, float(np.max(err / a)))
    return worst, time.perf_counter() - t0


@pytest.mark.parametrize("ci", [0, 1])
def test_full_size_workloads_every_route(ci):
    inp = synth.make_moe_inputs(ci)
    c = inp.config
    print("moe full-size", c.name, flush=True)
    p = params(c.tokens, c.top_k, c.n, c.K, c.experts)
    run = Run(inp.x, inp.blocks, inp.ids, p)
    y = run.plain()  # decode: fp32 schedule; prefill (512 tokens, top_k 6): matrix cores
    assert run.flagged() == 0 and np.all(np.isfinite(y))
    worst, sec = _check_every_route(y, inp, bf16=(ci == 1))
    print("moe full-size %s: all %d routes x %d outputs, max |err|/A = %.3g (oracle %.1f s)" % (
        c.name, c.routes, c.n, worst, sec), flush=True)
