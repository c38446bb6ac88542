"""Pins of the CPU oracle to facts that do not come from the oracle itself.

The oracle restates the docs.rs source page of mlx-native 0.10.8,
tests/deepseek_q2_k.rs. Each test here checks it against something fixed by
that page or by mathematics: hand-decoded fixture values, numpy's independent
f16 conversion, invariants of the block format, exact rational arithmetic and
torch's bf16 rounding. A plausible slip in the oracle (a wrong nibble, shift,
byte index, sign or accumulation) fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

QK_K, BB = 256, 84


def _rng(seed=7):
    return np.random.Generator(np.random.PCG64(seed))


def _f16_bits(v):
    return int(np.float16(v).view(np.uint16))


def _set_d(blk, d_bits, dmin_bits):
    blk = blk.copy()
    blk[80], blk[81] = d_bits & 0xFF, d_bits >> 8
    blk[82], blk[83] = dmin_bits & 0xFF, dmin_bits >> 8
    return blk


def _random_block(rng, wide=False):
    """A random block; wide=True draws d and dmin from all finite f16 patterns."""
    blk = rng.integers(0, 256, BB, dtype=np.uint8)
    if not wide:
        blk = _set_d(blk, _f16_bits(rng.uniform(0.01, 0.2)), _f16_bits(rng.uniform(0, 0.1)))
    else:
        def finite():
            while True:
                b = int(rng.integers(0, 1 << 16))
                if (b >> 10) & 0x1F != 31:
                    return b
        blk = _set_d(blk, finite(), finite())
    return blk


# ---------------------------------------------------------------- f16 decode

def test_f16_decode_all_65536_patterns_match_numpy():
    bits = np.arange(1 << 16, dtype=np.uint16)
    mine = oracle.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---------------------------------------------------------------- page fixture

def test_page_block5_bytes_match_hand_derivation(golden):
    blk = synth.page_block(5)
    for off, hexv in golden("block5_bytes.txt"):
        assert blk[int(off)] == int(hexv, 16), off


def test_page_block5_hand_decoded_values(golden):
    out = oracle.dequant_block(synth.page_block(5))
    for idx, val, *_ in golden("block5_hand_decode.txt"):
        if idx == "SUM":
            continue
        assert out[int(idx)] == np.float32(float(val)), idx
    # The page also asserts the decoded fixture has both signs.
    assert (out < 0).any() and (out > 0).any()


def test_page_block5_sum_of_decoded_values(golden):
    # The hand-derived total (per sub-block d*sc*sum(q) - 16*dmin*mn, golden file) against the oracle's
    # 256 decoded values summed exactly: a dropped element, sub-block or min term would move it.
    want = [float(v) for tag, v, *_ in golden("block5_hand_decode.txt") if tag == "SUM"]
    out = oracle.dequant_block(synth.page_block(5))
    assert want == [256.875]
    assert sum(Fraction(float(v)) for v in out) == Fraction(2055, 8)


def test_page_block5_decode_is_exact_sixteenths():
    # d = 1/8 and dmin = 1/16, so every value is (2*sc*q - mn)/16 exactly.
    out = oracle.dequant_block(synth.page_block(5)).astype(np.float64)
    assert np.all(out * 16 == np.round(out * 16))
    assert out.min() >= -15 / 16 and out.max() <= 2 * 15 * 3 / 16


# ---------------------------------------------------------------- format invariants

@pytest.mark.parametrize("seed", range(6))
def test_loop_order_equals_closed_form_map(seed):
    rng = _rng(100 + seed)
    for _ in range(20):
        blk = _random_block(rng, wide=bool(seed % 2))
        loop = oracle.dequant_block(blk)
        closed = np.array([oracle.dequant_element(blk, e) for e in range(QK_K)], dtype=np.float32)
        assert np.array_equal(loop.view(np.uint32), closed.view(np.uint32))


def _field_values(blk):
    d = np.float16(np.frombuffer(blk[80:82].tobytes(), "<f2")[0]).astype(np.float64)
    dmin = np.float16(np.frombuffer(blk[82:84].tobytes(), "<f2")[0]).astype(np.float64)
    return d, dmin


def test_all_zero_codes_give_minus_dmin_times_min():
    rng = _rng(1)
    for _ in range(20):
        blk = _random_block(rng)
        blk[16:80] = 0
        d, dmin = _field_values(blk)
        out = oracle.dequant_block(blk)
        for e in range(QK_K):
            mn = blk[e // 16] >> 4
            assert out[e] == np.float32(-(dmin * mn))


def test_all_three_codes_round_once_from_exact_value():
    # q = 3 everywhere: w = RN_f32(3*d*sc - dmin*mn) computed exactly in f64
    # (d*sc*3 and dmin*mn are exact in f64, so only the f32 rounding remains).
    rng = _rng(2)
    for wide in (False, True):
        for _ in range(30):
            blk = _random_block(rng, wide)
            blk[16:80] = 0xFF
            d, dmin = _field_values(blk)
            out = oracle.dequant_block(blk)
            for e in range(QK_K):
                sc, mn = blk[e // 16] & 15, blk[e // 16] >> 4
                exact = 3 * d * sc - dmin * mn
                assert out[e] == np.float32(exact) or (np.isnan(out[e]) and np.isnan(exact))


def test_zero_scale_nibble_gives_constant_minus_min():
    rng = _rng(3)
    blk = _random_block(rng)
    blk[0:16] &= 0xF0
    d, dmin = _field_values(blk)
    out = oracle.dequant_block(blk)
    for e in range(QK_K):
        assert out[e] == np.float32(-(dmin * (blk[e // 16] >> 4)))


def test_zero_min_nibble_gives_non_negative_multiples_of_d():
    rng = _rng(4)
    blk = _random_block(rng)
    blk[0:16] &= 0x0F
    d, _ = _field_values(blk)
    out = oracle.dequant_block(blk).astype(np.float64)
    assert np.all(out >= 0)
    for e in range(QK_K):
        ratio = out[e] / (d * (blk[e // 16] & 15)) if blk[e // 16] & 15 else 0.0
        assert ratio in (0.0, 1.0, 2.0, 3.0)


def test_zero_d_and_dmin_give_positive_zero():
    rng = _rng(5)
    blk = _set_d(_random_block(rng), 0, 0)
    out = oracle.dequant_block(blk)
    assert np.all(out.view(np.uint32) == 0)


def test_each_code_bit_moves_exactly_one_element():
    # Code byte i, bit b holds element 128*(i//32) + 32*(b//2) + i%32; bit 0 of
    # the pair is worth 1 and bit 1 worth 2 units of d*sc.
    rng = _rng(6)
    blk = _random_block(rng)
    blk[0:16] = (blk[0:16] & 0xF0) | 0x07      # every scale nibble non-zero
    d, _ = _field_values(blk)
    base = oracle.dequant_block(blk).astype(np.float64)
    for i in range(64):
        for b in range(8):
            alt = blk.copy()
            alt[16 + i] ^= 1 << b
            diff = oracle.dequant_block(alt).astype(np.float64) - base
            changed = np.flatnonzero(diff)
            e = 128 * (i // 32) + 32 * (b // 2) + i % 32
            assert changed.tolist() == [e], (i, b)
            sign = 1 if alt[16 + i] & (1 << b) else -1
            unit = d * 7 * (1 if b % 2 == 0 else 2)
            assert abs(diff[e] - sign * unit) <= 1e-6 * abs(unit)


def test_scale_byte_bits_touch_only_their_sixteen_elements():
    rng = _rng(7)
    blk = _random_block(rng)
    base = oracle.dequant_block(blk)
    for s in range(16):
        for b in range(8):
            alt = blk.copy()
            alt[s] ^= 1 << b
            changed = np.flatnonzero(oracle.dequant_block(alt) != base)
            assert set(changed.tolist()) <= set(range(16 * s, 16 * s + 16)), (s, b)
            if b >= 4:   # a min-nibble bit moves all 16 (dmin != 0 here)
                assert len(changed) == 16


def test_d_and_dmin_bytes_are_little_endian_f16_at_80_and_82():
    blk = synth.page_block(1)
    blk = _set_d(blk, _f16_bits(2.0), _f16_bits(0.0))
    blk[0:16] = 0x01                     # sc 1, mn 0 everywhere
    blk[16:80] = 0x55                    # code 1 at every position
    assert np.all(oracle.dequant_block(blk) == 2.0)
    blk = _set_d(blk, _f16_bits(0.0), _f16_bits(0.5))
    blk[0:16] = 0x30                     # sc 0, mn 3
    assert np.all(oracle.dequant_block(blk) == -1.5)


# ---------------------------------------------------------------- malformed input

def test_dequantize_rejects_malformed_buffers_like_the_page():
    blk = synth.page_block(1)
    with pytest.raises(oracle.OracleError):
        oracle.dequantize(blk[:BB - 1], QK_K)
    with pytest.raises(oracle.OracleError):
        oracle.dequantize(blk, QK_K - 1)
    assert oracle.dequantize(blk, QK_K).shape == (QK_K,)


# ---------------------------------------------------------------- matmul

def _exact_matmul(x, w_dense):
    M, K = x.shape
    N = w_dense.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    a = [[Fraction(0)] * N for _ in range(M)]
    xf = [[Fraction(float(v)) for v in row] for row in x]
    wf = [[Fraction(float(v)) for v in row] for row in w_dense]
    for m in range(M):
        for n in range(N):
            s = sa = Fraction(0)
            for k in range(K):
                p = xf[m][k] * wf[n][k]
                s += p
                sa += abs(p)
            y[m][n], a[m][n] = s, sa
    return y, a


@pytest.mark.parametrize("M,N,K", [(1, 3, 256), (3, 2, 512)])
def test_matmul_matches_exact_rational_brute_force(M, N, K):
    rng = _rng(M * 10 + N)
    blocks = synth.random_blocks(rng, N * K // QK_K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w_dense = oracle.dequantize(blocks).reshape(N, K)
    y, a = oracle.matmul(x, blocks, M, N, K)
    ey, ea = _exact_matmul(x, w_dense)
    for m in range(M):
        for n in range(N):
            bound = 2 * K * 2.0 ** -53 * float(ea[m][n])
            assert abs(Fraction(float(y[m, n])) - ey[m][n]) <= Fraction(bound)
            assert abs(Fraction(float(a[m, n])) - ea[m][n]) <= Fraction(bound)


def test_matmul_row_n_uses_blocks_of_row_n():
    # One-hot activations pick out single weights: y[m, n] = w[n, k].
    rng = _rng(11)
    M, N, K = 4, 5, 768
    blocks = synth.random_blocks(rng, N * K // QK_K)
    w_dense = oracle.dequantize(blocks).reshape(N, K)
    ks = [0, 255, 256 + 17, K - 1]
    x = np.zeros((M, K), dtype=np.float32)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    y, _ = oracle.matmul(x, blocks, M, N, K)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m].astype(np.float32), w_dense[:, k])


def test_matmul_results_do_not_depend_on_thread_count():
    inp = synth.make_inputs(0)
    c = inp.config
    y1, a1 = oracle.matmul(inp.x, inp.blocks, c.M, c.N, c.K, nthreads=1)
    y4, a4 = oracle.matmul(inp.x, inp.blocks, c.M, c.N, c.K, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(a1, a4)


def test_page_dense_fixture_cpu_dot_within_page_tolerance():
    # fn run_dense(1): 8 rows block(row + 1), x = input(1); the page compares
    # its GPU result against cpu_dot with abs tolerance 2e-4.
    blocks = np.concatenate([synth.page_block(r + 1) for r in range(8)])
    x = synth.page_input(1).reshape(1, QK_K)
    y64, a = oracle.matmul(x, blocks, 1, 8, QK_K)
    y32 = oracle.matmul_f32seq(x, blocks, 1, 8, QK_K)
    w_dense = oracle.dequantize(blocks).reshape(8, QK_K)
    ey, _ = _exact_matmul(x, w_dense)
    for n in range(8):
        assert abs(float(y64[0, n]) - float(ey[0][n])) <= 1e-12 * a[0, n]
        # f32 left-to-right summation: |error| <= K * 2^-24 * sum|x*w| (to first order).
        assert abs(float(y32[0, n]) - float(ey[0][n])) <= (QK_K + 1) * 2.0 ** -24 * a[0, n]
    assert np.all(np.abs(y32 - y64) <= 2e-4)


def test_matmul_rejects_bad_shapes():
    with pytest.raises(oracle.OracleError):
        oracle.matmul(np.zeros((1, 100), np.float32), np.zeros(84, np.uint8), 1, 1, 100)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_ties_to_even_and_specials():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {
        one + ulp / 2: one,                       # tie, even below
        one + 3 * ulp / 2: one + 2 * ulp,         # tie, even above
        one + ulp / 2 + 2.0 ** -20: one + ulp,    # just above the tie
        -(one + ulp / 2): -one,
        0.0: 0.0,
        float("inf"): float("inf"),
    }
    got = oracle.bf16_round(list(cases))
    assert np.array_equal(got, np.array(list(cases.values()), dtype=np.float32))
    assert np.isnan(oracle.bf16_round([float("nan")])[0])
    assert oracle.bf16_round([-0.0]).view(np.uint32)[0] == 0x80000000


def test_bf16_round_matches_torch_on_random_values():
    torch = pytest.importorskip("torch")
    rng = _rng(12)
    v = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                        rng.integers(0, 1 << 32, 3000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.bf16_round(v).view(np.uint32), ref.view(np.uint32))


def test_bf16_matmul_equals_f64_product_of_rounded_operands():
    rng = _rng(13)
    M, N, K = 2, 3, 256
    blocks = synth.random_blocks(rng, N)
    x = rng.standard_normal((M, K)).astype(np.float32)
    y, _ = oracle.matmul(x, blocks, M, N, K, bf16_operands=True)
    wb = oracle.bf16_round(oracle.dequantize(blocks)).reshape(N, K).astype(np.float64)
    xb = oracle.bf16_round(x).reshape(M, K).astype(np.float64)
    ey, ea = _exact_matmul(xb, wb)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - ey[m][n]) <= Fraction(2 * K * 2.0 ** -53 * float(ea[m][n]))


# ---------------------------------------------------------------- gather

def test_gather_page_fixture_and_bad_id():
    vocab = 3
    table = np.concatenate([synth.page_block(r + 2) for r in range(vocab)])
    out = oracle.gather(table, [2, 0], vocab, QK_K, 2)
    assert np.array_equal(out[0], oracle.dequant_block(synth.page_block(4)))
    assert np.array_equal(out[1], oracle.dequant_block(synth.page_block(2)))
    with pytest.raises(oracle.OracleError):
        oracle.gather(table, [2, vocab], vocab, QK_K, 2)


def test_gather_duplicates_and_multi_block_rows():
    rng = _rng(14)
    vocab, dim = 5, 768
    table = synth.random_blocks(rng, vocab * dim // QK_K)
    ids = [4, 4, 0, 2]
    out = oracle.gather(table, ids, vocab, dim, len(ids), nthreads=3)
    dense = oracle.dequantize(table).reshape(vocab, dim)
    assert np.array_equal(out, dense[ids])


def test_batched_matmul_is_independent_products_with_exact_rationals():
    # The page defines the batched mat-vec as separate single-matrix products; check the
    # oracle's stacking against exact rational arithmetic on a tiny case.
    rng = _rng(43)
    batches, M, N, K = 3, 2, 2, 256
    blocks = synth.random_blocks(rng, batches * N)
    x = rng.standard_normal((batches, M, K)).astype(np.float32)
    y, a = oracle.matmul_batched(x, blocks, batches, M, N, K)
    for b in range(batches):
        for n in range(N):
            blk = blocks[(b * N + n) * BB:(b * N + n + 1) * BB]
            w = oracle.dequant_block(blk)
            for m in range(M):
                exact = sum(Fraction(float(x[b, m, k])) * Fraction(float(w[k])) for k in range(K))
                assert abs(Fraction(float(y[b, m, n])) - exact) <= Fraction(1, 10**12) * (1 + abs(exact))
