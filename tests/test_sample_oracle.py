"""Pins of the argmax / threshold-candidate oracle (CPU only).

The operation is the docs.rs source page of mlx-native 0.9.5,
src/mlx_native/ops/gpu_sample.rs: per slot the first maximum (lower index wins
ties) and every index whose logit is >= top1 - 0.5f, with a count that may
exceed the capacity and an overflow flag. The oracle is checked against
numpy's own argmax and comparisons on NaN-free data, and against hand-worked
rows for ties, NaN, infinities and the threshold boundary.
"""
import numpy as np
import pytest

import oracle


def _one(row, cap):
    idx, val, cnt, ovf, ids = oracle.argmax_candidates(np.asarray(row, np.float32), 1, len(row), cap)
    return int(idx[0]), float(val[0]), int(cnt[0]), int(ovf[0]), ids[0].tolist()


def test_matches_numpy_on_random_rows():
    rng = np.random.Generator(np.random.PCG64(61))
    n_slots, vocab, cap = 6, 5000, 16
    x = rng.standard_normal((n_slots, vocab)).astype(np.float32) * 3
    x[2, 17] = x[2, 4000] = x[2].max() + 1  # a tie: the lower index wins
    idx, val, cnt, ovf, ids = oracle.argmax_candidates(x, n_slots, vocab, cap)
    for s in range(n_slots):
        assert idx[s] == np.argmax(x[s])                         # numpy: first occurrence
        assert val[s] == x[s].max()
        hit = np.flatnonzero(x[s] >= np.float32(x[s].max()) - np.float32(0.5))
        assert cnt[s] == hit.size and ovf[s] == (hit.size > cap)
        assert np.array_equal(ids[s], hit[:cap])
    assert idx[2] == 17


def test_threshold_boundary_is_inclusive_in_f32():
    top = np.float32(3.0)
    thr = top - np.float32(0.5)
    row = [0.0, thr, np.nextafter(thr, np.float32(-np.inf)), top, 2.75]
    assert _one(row, 8) == (3, 3.0, 3, 0, [1, 3, 4])


def test_ties_take_the_lowest_index_and_count_all_of_them():
    assert _one([1.0, 5.0, 5.0, 4.6, 5.0], 8) == (1, 5.0, 4, 0, [1, 2, 3, 4])


def test_overflow_keeps_the_first_cap_ids():
    row = np.zeros(100, np.float32)
    idx, val, cnt, ovf, ids = _one(row, 7)
    assert (idx, val, cnt, ovf) == (0, 0.0, 100, 1) and ids == list(range(7))


def test_nan_in_column_zero_stays_the_answer_and_leaves_no_candidates():
    idx, val, cnt, ovf, ids = _one([np.nan, 1.0, 9.0], 4)
    assert idx == 0 and np.isnan(val) and cnt == 0 and ovf == 0 and ids == []


def test_nan_elsewhere_is_passed_over():
    assert _one([1.0, np.nan, 9.0, np.nan], 4) == (2, 9.0, 1, 0, [2])


def test_infinities():
    assert _one([-np.inf, -np.inf, -np.inf], 2) == (0, -np.inf, 3, 1, [0, 1])
    assert _one([1.0, np.inf, 2.0, np.inf], 4) == (1, np.inf, 2, 0, [1, 3])


def test_zero_sizes_are_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.argmax_candidates(np.zeros(0, np.float32), 1, 0, 4)
