"""Pins for the oracle's canonical order and top-k select (CPU only).

The oracle's top-k is pinned to things other than itself: O(V^2) brute-force ranks,
numpy's stable sort, closed forms (all-equal rows give [0, k); k = 1 is the first
argmax; k >= V keeps every index) and the short-row -1 padding of vLLM PR #55122
("Test plan").
"""
import math

import numpy as np
import pytest

import oracle


def brute_ranks(x):
    """rank_i = #{j : x_j > x_i or (x_j == x_i and j < i)} -- no sorting involved."""
    n = len(x)
    return [sum(1 for j in range(n) if x[j] > x[i] or (x[j] == x[i] and j < i)) for i in range(n)]


def rows_for_pins(seed, count=150, v=16):
    rng = np.random.default_rng(seed)
    rows = []
    for r in range(count):
        kind = r % 5
        if kind == 0:
            x = rng.standard_normal(v)
        elif kind == 1:
            x = rng.integers(-2, 3, size=v).astype(np.float64)          # heavy ties
        elif kind == 2:
            x = rng.choice([0.0, -0.0, 1.0, -1.0], size=v)               # signed zeros
        elif kind == 3:
            x = rng.standard_normal(v) * 1e30
        else:
            x = rng.standard_normal(v)
            x[rng.integers(0, v, 3)] = -np.inf
            x[rng.integers(0, v)] = np.inf
        rows.append(x.astype(np.float32))
    return rows


def test_canonical_order_matches_brute_force_ranks():
    for x in rows_for_pins(101):
        xf = oracle.row_floats(x)
        order = oracle.canonical_order(xf)
        ranks = brute_ranks(xf)
        assert [order.index(i) for i in range(len(xf))] == ranks


def test_canonical_order_matches_numpy_stable_sort():
    rng = np.random.default_rng(7)
    for _ in range(20):
        x = np.round(rng.standard_normal(500), 1).astype(np.float32)
        x[rng.integers(0, 500, 20)] = -0.0
        xf = oracle.row_floats(x)
        ref = np.argsort(-x.astype(np.float64), kind="stable").tolist()
        assert oracle.canonical_order(xf) == ref


def test_signed_zero_ties_by_index():
    x = np.array([-0.0, 0.0, -0.0, 0.0], np.float32)
    assert oracle.canonical_order(oracle.row_floats(x)) == [0, 1, 2, 3]
    st, idx = oracle.topk_select_row(x, 2, 4)
    assert st == 0 and idx == [0, 1, -1, -1]


def test_topk_matches_brute_force_rank_set():
    rng = np.random.default_rng(3)
    for x in rows_for_pins(202):
        xf = oracle.row_floats(x)
        ranks = brute_ranks(xf)
        k = int(rng.integers(1, 17))
        st, idx = oracle.topk_select_row(x, k, 16)
        assert st == 0
        want = sorted(i for i in range(16) if ranks[i] < k)
        assert idx == want + [-1] * (16 - len(want))


@pytest.mark.parametrize("k", [1, 7, 100, 511])
def test_topk_all_equal_is_prefix_of_indices(k):
    x = np.full(512, 3.25, np.float32)
    st, idx = oracle.topk_select_row(x, k, 512)
    assert st == 0 and idx[:k] == list(range(k)) and all(v == -1 for v in idx[k:])


def test_topk_k1_is_first_argmax():
    rng = np.random.default_rng(9)
    for _ in range(50):
        x = rng.integers(-3, 4, size=40).astype(np.float32)
        st, idx = oracle.topk_select_row(x, 1, 1)
        assert st == 0 and idx == [int(np.argmax(x))]


def test_topk_short_row_pads_minus_one():
    x = np.arange(10, dtype=np.float32)
    st, idx = oracle.topk_select_row(x, 50, 64)
    assert st == 0 and idx == list(range(10)) + [-1] * 54


def test_topk_distinct_values_match_argpartition_set():
    rng = np.random.default_rng(11)
    for _ in range(20):
        x = rng.permutation(4000).astype(np.float32) * 0.5
        k = int(rng.integers(1, 300))
        st, idx = oracle.topk_select_row(x, k, k)
        assert st == 0
        assert idx == sorted(np.argpartition(-x, k - 1)[:k].tolist())


def test_topk_status_codes():
    x = np.zeros(8, np.float32)
    assert oracle.topk_select_row(x, 0, 4)[0] == oracle.STATUS_BAD_K
    assert oracle.topk_select_row(x, 5, 4)[0] == oracle.STATUS_BAD_K       # 5 > k_max
    assert oracle.topk_select_row(x[:3], 5, 4)[0] == 0                      # short row fits
    y = x.copy()
    y[3] = np.nan
    st, idx = oracle.topk_select_row(y, 2, 4)
    assert st == oracle.STATUS_NONFINITE and idx == [-1] * 4
    z = np.array([1.0, np.inf, -np.inf, 2.0], np.float32)                  # +-inf are keys
    assert oracle.topk_select_row(z, 2, 2) == (0, [1, 3])
    assert oracle.topk_select_row(z, 4, 4) == (0, [0, 1, 2, 3])


def test_batched_topk_shapes():
    x = np.random.default_rng(0).standard_normal((3, 20)).astype(np.float32)
    st, out = oracle.topk_select(x, np.array([1, 5, 20]), 20)
    assert st.tolist() == [0, 0, 0] and out.shape == (3, 20)
    assert (out[0, 1:] == -1).all() and (out[2] == np.arange(20)).all()
    assert math.isfinite(float(x[1, out[1, 0]]))
