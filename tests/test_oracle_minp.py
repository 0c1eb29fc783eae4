"""Pins of the oracle's min-p step (after top-k and top-p).

min-p keeps the tokens whose probability is at least min_p times the largest. Pinned by
closed forms (all-equal rows, two-token rows), scipy's softmax (probability ratios computed
by a library routine), the identity at min_p = 0, the prefix and monotonicity invariants,
and the status of invalid values.
"""
import math

import numpy as np
import pytest

import oracle


def test_min_p_zero_is_identity():
    rng = np.random.default_rng(11)
    for _ in range(20):
        row = (rng.standard_normal(300) * 2).astype(np.float32)
        a = oracle.topp_row(row, 100, 0.9, 1.0)
        b = oracle.topp_minp_row(row, 100, 0.9, 1.0, 0.0)
        assert b.kept == a.kept and b.kept_ids == a.kept_ids


def test_all_equal_row_keeps_everything():
    row = np.full(50, 1.5, np.float32)
    for mp in (0.01, 0.5, 1.0):
        res = oracle.topp_minp_row(row, 50, 1.0, 1.0, mp)
        assert res.kept == 50


def test_two_tokens_closed_form():
    # weights 1 and exp(-d / T): the second stays iff exp(-d / T) >= min_p
    for d, t, mp in ((1.0, 1.0, 0.3), (1.0, 1.0, 0.4), (2.0, 0.5, 0.02), (2.0, 0.5, 0.018), (0.5, 2.0, 0.75)):
        row = np.array([0.0, -d], np.float32)
        res = oracle.topp_minp_row(row, None, None, t, mp)
        keep2 = math.exp(-float(np.float32(d)) / t) >= mp
        assert res.kept == (2 if keep2 else 1), (d, t, mp)


def test_probability_ratio_against_scipy_softmax():
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(12)
    for _ in range(30):
        v = int(rng.integers(5, 400))
        row = (rng.standard_normal(v) * rng.uniform(0.5, 4)).astype(np.float32)
        t = float(np.float32(rng.uniform(0.3, 2.0)))
        k = int(rng.integers(1, v + 1))
        mp = float(np.float32(rng.uniform(0.001, 0.5)))
        res = oracle.topp_minp_row(row, k, None, t, mp)
        prob = special.softmax(row.astype(np.float64) / t)
        keep = [i for i in res.topk if prob[i] >= mp * prob.max() * (1 - 1e-12)]
        # the library's probabilities agree with the kept set away from the boundary
        if not res.minp_ambiguous:
            assert sorted(res.kept_ids) == sorted(keep)


def test_prefix_monotone_and_keeps_max():
    rng = np.random.default_rng(13)
    row = (rng.standard_normal(500) * 3).astype(np.float32)
    prev = None
    for mp in (0.0, 0.001, 0.01, 0.1, 0.5, 1.0):
        res = oracle.topp_minp_row(row, 400, 0.95, 1.2, mp)
        assert res.kept >= 1 and res.kept_ids[0] == int(np.argmax(row))
        assert res.kept_ids == res.order[: res.kept]
        if prev is not None:
            assert res.kept <= prev
        prev = res.kept


def test_invalid_min_p_status():
    row = np.zeros(8, np.float32)
    for bad in (-0.1, 1.5, float("nan")):
        assert oracle.topp_minp_row(row, 4, 0.9, 1.0, bad).status == oracle.STATUS_BAD_MINP
    # the other parameters are checked first
    assert oracle.topp_minp_row(row, 0, 0.9, 1.0, -1.0).status == oracle.STATUS_BAD_K


def test_sampling_stays_in_min_p_set():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((20, 64)) * 2).astype(np.float32)
    k = np.full(20, 64)
    p = np.full(20, 0.99, np.float32)
    t = np.ones(20, np.float32)
    mp = np.full(20, 0.2, np.float32)
    seeds = rng.integers(0, 2 ** 63, 20, dtype=np.uint64)
    for r, res in enumerate(oracle.sample_rows_minp(x, k, p, t, mp, seeds)):
        assert res.token in res.topp.kept_ids
