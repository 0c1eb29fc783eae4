"""Pins of the oracle's sparse-indexer top-k (per-row lengths, value or index order, id
offsets): brute-force ranks on tiny rows, numpy's lexsort for the value order, length
clamping, empty and short rows, NaN past the valid prefix, and the offsets."""
import itertools

import numpy as np
import pytest

import oracle


def brute_topk(vals, k):
    """The k ids that no other id outranks more than k-1 times: rank = #(y > x or y == x and j < i)."""
    n = len(vals)
    ranks = [sum(1 for j in range(n) if vals[j] > vals[i] or (vals[j] == vals[i] and j < i)) for i in range(n)]
    return [i for i in range(n) if ranks[i] < k], ranks


def test_brute_force_with_lengths_both_orders():
    rng = np.random.default_rng(21)
    for _ in range(300):
        v = int(rng.integers(1, 12))
        row = rng.integers(-3, 4, v).astype(np.float32)     # many ties
        length = int(rng.integers(-2, v + 3))
        k = int(rng.integers(1, 14))
        n = max(0, min(length, v))
        chosen, ranks = brute_topk([float(a) for a in row[:n]], k)
        st, out_i = oracle.topk_select_rows_row(row, length, k, 16, oracle.ORDER_INDEX)
        st2, out_v = oracle.topk_select_rows_row(row, length, k, 16, oracle.ORDER_VALUE)
        assert st == 0 and st2 == 0
        ke = min(k, n)
        assert out_i[:ke] == sorted(chosen) and all(o == -1 for o in out_i[ke:])
        assert out_v[:ke] == sorted(chosen, key=lambda i: ranks[i])


def test_value_order_matches_numpy_lexsort():
    rng = np.random.default_rng(22)
    for _ in range(20):
        v = int(rng.integers(50, 3000))
        row = np.round(rng.standard_normal(v), 2).astype(np.float32)
        length = int(rng.integers(1, v + 1))
        k = int(rng.integers(1, 300))
        st, out = oracle.topk_select_rows_row(row, length, k, 300, oracle.ORDER_VALUE, offset=1000)
        pre = row[:length].astype(np.float64)
        want = np.lexsort((np.arange(length), -pre))[: min(k, length)]
        assert st == 0 and out[: len(want)] == [1000 + int(i) for i in want]


def test_clamping_short_rows_and_nan_past_length():
    row = np.array([5, 1, np.nan, 7], np.float32)
    assert oracle.topk_select_rows_row(row, 2, 3, 4)[1] == [0, 1, -1, -1]       # NaN past n ignored
    assert oracle.topk_select_rows_row(row, 3, 1, 4)[0] == oracle.STATUS_NONFINITE
    assert oracle.topk_select_rows_row(row, 0, 3, 4) == (0, [-1, -1, -1, -1])   # empty row
    assert oracle.topk_select_rows_row(row, -5, 3, 4) == (0, [-1, -1, -1, -1])
    ok = np.array([5, 1, 2, 7], np.float32)
    assert oracle.topk_select_rows_row(ok, 99, 2, 4)[1] == [0, 3, -1, -1]        # clamped to the row
    assert oracle.topk_select_rows_row(ok, 99, 2, 4, oracle.ORDER_VALUE)[1] == [3, 0, -1, -1]
    assert oracle.topk_select_rows_row(ok, 4, 0, 4)[0] == oracle.STATUS_BAD_K
    assert oracle.topk_select_rows_row(ok, 4, 4, 3)[0] == oracle.STATUS_BAD_K      # k_eff > k_max
    assert oracle.topk_select_rows_row(ok, 2, 4, 3)[0] == 0                        # k_eff = 2 fits


def test_whole_row_index_order_is_plain_topk():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((5, 400)).astype(np.float32)
    k = rng.integers(1, 400, 5)
    st, out = oracle.topk_select_rows(x, None, k, 400)
    st0, out0 = oracle.topk_select(x, k, 400)
    assert np.array_equal(st, st0) and np.array_equal(out, out0)
