"""Pins of the oracle's expert-routed product (CPU only).

The definition is on the docs.rs source page of mlx-native 0.10.8,
tests/deepseek_q2_k.rs: fn run_expert builds expert e's row r from
fn block(e * n + r + 1), routes token t's slot s to expert (3 t + s) mod
experts and expects out[route, row] = cpu_dot(decoded row, x[token]) within
2e-4 (1e-2 for the matrix-multiply schedules); the slotted down-projection test
feeds one activation row per route and requires the slotted run to equal the
flattened run (n_tokens = tokens * top_k, top_k = 1) byte for byte.

The checks below tie oracle.matmul_id to things other than itself: exact
rational arithmetic on tiny cases, the page's own f32 expectation on its
fixtures, the dense product when every route picks one expert, and the
structural facts (slotted = flattened, padding between experts unread, bad ids
give NaN rows).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

QK_K, BB = 256, 84


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _cpu_dot(w_row, x_row):
    """The page's cpu_dot: f32 products summed left to right in f32 (numpy cumsum is sequential)."""
    return np.cumsum(w_row.astype(np.float32) * x_row.astype(np.float32), dtype=np.float32)[-1]


@pytest.mark.parametrize("tokens,top_k,experts", [(2, 2, 3), (33, 6, 8)])
def test_page_expert_fixture_within_page_tolerance(tokens, top_k, experts):
    n = 8
    w = synth.page_expert_weights(experts, n)
    x = synth.page_input(tokens).reshape(tokens, QK_K)
    ids = synth.page_routes(tokens, top_k, experts)
    y, a, bad = oracle.matmul_id(x, w, ids, tokens, top_k, n, QK_K, experts, n * BB)
    assert bad == 0
    dec = oracle.dequantize(w).reshape(experts, n, QK_K)
    for r, e in enumerate(ids.tolist()):
        t = r // top_k
        for row in range(n):
            want = _cpu_dot(dec[e, row], x[t])
            assert abs(y[r, row] - float(want)) <= 2e-4
            # f32 left-to-right summation error bound against the f64 oracle.
            assert abs(y[r, row] - float(want)) <= (QK_K + 1) * 2.0 ** -24 * a[r, row]


def _exact(x_rows, w_rows):
    xf = [Fraction(float(v)) for v in x_rows]
    s = sa = Fraction(0)
    for xv, wv in zip(xf, (Fraction(float(v)) for v in w_rows)):
        s += xv * wv
        sa += abs(xv * wv)
    return s, sa


@pytest.mark.parametrize("slotted", [False, True])
def test_exact_rational_brute_force(slotted):
    tokens, top_k, experts, n, K = 3, 2, 3, 2, 512
    rng = _rng(61 + slotted)
    rb = (K // QK_K) * BB
    w = synth.random_blocks(rng, experts * n * K // QK_K)
    rows_x = tokens * top_k if slotted else tokens
    x = rng.standard_normal((rows_x, K)).astype(np.float32)
    ids = np.array([2, 0, 1, 1, 0, 2], dtype=np.uint32)  # token 1 sends both slots to expert 1
    y, a, bad = oracle.matmul_id(x, w, ids, tokens, top_k, n, K, experts, n * rb, slotted=slotted)
    assert bad == 0
    dec = oracle.dequantize(w).reshape(experts, n, K)
    for r in range(tokens * top_k):
        xr = r if slotted else r // top_k
        for row in range(n):
            es, ea = _exact(x[xr], dec[ids[r], row])
            bound = 2 * K * 2.0 ** -53 * float(ea)
            assert abs(Fraction(float(y[r, row])) - es) <= Fraction(bound)
            assert abs(Fraction(float(a[r, row])) - ea) <= Fraction(bound)


def test_single_expert_top1_reduces_to_the_dense_product():
    tokens, experts, n, K = 5, 4, 3, 768
    rng = _rng(62)
    rb = (K // QK_K) * BB
    w = synth.random_blocks(rng, experts * n * K // QK_K)
    x = rng.standard_normal((tokens, K)).astype(np.float32)
    for e in range(experts):
        ids = np.full(tokens, e, dtype=np.uint32)
        y, a, _ = oracle.matmul_id(x, w, ids, tokens, 1, n, K, experts, n * rb)
        yd, ad = oracle.matmul(x, w[e * n * rb:(e + 1) * n * rb], tokens, n, K)
        assert np.array_equal(y, yd) and np.array_equal(a, ad)


def test_slotted_equals_flattened_and_repeated_rows_equal_plain():
    tokens, top_k, experts, n, K = 7, 3, 5, 4, 512
    rng = _rng(63)
    rb = (K // QK_K) * BB
    w = synth.random_blocks(rng, experts * n * K // QK_K)
    ids = synth.random_routes(rng, tokens, top_k, experts)
    xs = rng.standard_normal((tokens * top_k, K)).astype(np.float32)
    ys, _, _ = oracle.matmul_id(xs, w, ids, tokens, top_k, n, K, experts, n * rb, slotted=True)
    yf, _, _ = oracle.matmul_id(xs, w, ids, tokens * top_k, 1, n, K, experts, n * rb)
    assert np.array_equal(ys, yf)
    # One activation row per token, repeated per slot, is the plain routing.
    xt = rng.standard_normal((tokens, K)).astype(np.float32)
    yp, _, _ = oracle.matmul_id(xt, w, ids, tokens, top_k, n, K, experts, n * rb)
    yr, _, _ = oracle.matmul_id(np.repeat(xt, top_k, axis=0), w, ids, tokens, top_k, n, K, experts, n * rb,
                                slotted=True)
    assert np.array_equal(yp, yr)


def test_padding_between_experts_is_never_read():
    tokens, top_k, experts, n, K = 4, 2, 3, 2, 256
    rng = _rng(64)
    rb = (K // QK_K) * BB
    w = synth.random_blocks(rng, experts * n)
    pad = 3 * BB + 4
    padded = np.full(experts * (n * rb + pad), 0xFF, dtype=np.uint8)  # 0xFFFF is an f16 NaN
    for e in range(experts):
        padded[e * (n * rb + pad):e * (n * rb + pad) + n * rb] = w[e * n * rb:(e + 1) * n * rb]
    x = rng.standard_normal((tokens, K)).astype(np.float32)
    ids = synth.random_routes(rng, tokens, top_k, experts)
    y0, _, _ = oracle.matmul_id(x, w, ids, tokens, top_k, n, K, experts, n * rb)
    y1, _, _ = oracle.matmul_id(x, padded, ids, tokens, top_k, n, K, experts, n * rb + pad)
    assert np.array_equal(y0, y1) and np.all(np.isfinite(y1))


def test_bad_ids_give_nan_rows_and_are_counted():
    tokens, top_k, experts, n = 3, 2, 3, 4
    w = synth.page_expert_weights(experts, n)
    x = synth.page_input(tokens).reshape(tokens, QK_K)
    ids = synth.page_routes(tokens, top_k, experts)
    ids[1] = experts
    ids[4] = 0xFFFFFFFF
    y, a, bad = oracle.matmul_id(x, w, ids, tokens, top_k, n, QK_K, experts, n * BB)
    assert bad == 2
    assert np.all(np.isnan(y[[1, 4]])) and np.all(np.isnan(a[[1, 4]]))
    good = [0, 2, 3, 5]
    yg, _, _ = oracle.matmul_id(x, w, synth.page_routes(tokens, top_k, experts), tokens, top_k, n, QK_K,
                                experts, n * BB)
    assert np.array_equal(y[good], yg[good])


def test_thread_count_does_not_change_results():
    tokens, top_k, experts, n = 9, 4, 8, 8
    w = synth.page_expert_weights(experts, n)
    x = synth.page_input(tokens).reshape(tokens, QK_K)
    ids = synth.page_routes(tokens, top_k, experts)
    y1, a1, _ = oracle.matmul_id(x, w, ids, tokens, top_k, n, QK_K, experts, n * BB, nthreads=1)
    y4, a4, _ = oracle.matmul_id(x, w, ids, tokens, top_k, n, QK_K, experts, n * BB, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(a1, a4)


def test_bf16_operands_round_both_sides():
    tokens, top_k, experts, n = 2, 2, 3, 8
    w = synth.page_expert_weights(experts, n)
    x = synth.page_input(tokens).reshape(tokens, QK_K)
    ids = synth.page_routes(tokens, top_k, experts)
    y, _, _ = oracle.matmul_id(x, w, ids, tokens, top_k, n, QK_K, experts, n * BB, bf16_operands=True)
    dec = oracle.bf16_round(oracle.dequantize(w)).reshape(experts, n, QK_K).astype(np.float64)
    xb = oracle.bf16_round(x).reshape(tokens, QK_K).astype(np.float64)
    for r, e in enumerate(ids.tolist()):
        want = dec[e] @ xb[r // top_k]
        assert np.allclose(y[r], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kw", [
    dict(K=300), dict(n_tokens=0), dict(top_k=0), dict(n_experts=0), dict(stride=8 * BB - 4),
])
def test_rejects_bad_shapes(kw):
    args = dict(n_tokens=2, top_k=2, n=8, K=QK_K, n_experts=3, stride=8 * BB)
    args.update(kw)
    w = synth.page_expert_weights(3, 8)
    x = np.zeros((max(args["n_tokens"], 1), args["K"]), np.float32)
    ids = np.zeros(max(args["n_tokens"] * args["top_k"], 1), np.uint32)
    with pytest.raises(oracle.OracleError):
        oracle.matmul_id(x, w, ids, args["n_tokens"], args["top_k"], args["n"], args["K"], args["n_experts"],
                         args["stride"])
