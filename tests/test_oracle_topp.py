"""Pins for the oracle's binary64 top-p (CPU only).

The top-p oracle follows "Split top-p numerical reference and conservative gate"
(section "Independent binary64 numerical reference"). Pinned here by exact subset
enumeration with rational arithmetic on V <= 12, closed forms (p = 1, all-equal rows
where the kept count is ceil(p*k), two-token rows, dominant tokens), a scipy logsumexp
cross-check of the normaliser, and the boundary invariants of the same section.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle


def exact_min_cardinality(w, p):
    """Smallest |S| over subsets S of the weights with sum(S) >= p * sum(w), in rationals."""
    fw = [Fraction(v) for v in w]
    target = Fraction(p) * sum(fw)
    for size in range(1, len(w) + 1):
        for comb in itertools.combinations(range(len(w)), size):
            if sum(fw[i] for i in comb) >= target:
                return size
    return len(w)


def test_brute_force_subset_enumeration_v12():
    rng = np.random.default_rng(5)
    checked = 0
    for r in range(120):
        v = 12
        if r % 3 == 0:
            x = rng.integers(-2, 3, size=v).astype(np.float32)
        else:
            x = (rng.standard_normal(v) * rng.uniform(0.3, 3.0)).astype(np.float32)
        k = int(rng.integers(1, v + 1))
        p = oracle.to_f32(rng.uniform(0.05, 0.999))
        t = oracle.to_f32(rng.uniform(0.25, 2.0))
        res = oracle.topp_row(x, k, p, t)
        assert res.status == 0
        if res.ambiguous:
            continue
        # the binary64 weights of K, summed exactly: the minimum cardinality must match
        assert res.kept == exact_min_cardinality(res.weights, p)
        # and the canonical prefix of that length must itself reach the target exactly
        fw = [Fraction(v_) for v_ in res.weights]
        assert sum(fw[: res.kept]) >= Fraction(p) * sum(fw)
        checked += 1
    assert checked > 100


@pytest.mark.parametrize("k,p,want", [(4, 0.5, 2), (4, 0.75, 3), (4, 0.25, 1), (10, 0.9, 9),
                                      (7, 0.5, 4), (1000, 0.999, 1000), (1000, 0.75, 750),
                                      (3, 1.0, 3)])
def test_all_equal_rows_keep_ceil_pk(k, p, want):
    # equal logits: every weight is exp(0) = 1, Z = k, so the count is ceil(p*k);
    # p*k integral checks the ">=" (reaching p keeps) convention; fp32(0.999) is slightly
    # above 0.999, so 1000 tokens need all 1000 (p is taken after fp32 conversion)
    x = np.full(k + 5, 1.5, np.float32)
    pf = oracle.to_f32(p)
    res = oracle.topp_row(x, k, pf, 1.0)
    assert res.kept == want == math.ceil(Fraction(pf) * k)
    assert res.kept_ids == list(range(want))


def test_p_one_keeps_all_of_topk():
    x = np.random.default_rng(0).standard_normal(300).astype(np.float32)
    res = oracle.topp_row(x, 77, 1.0, 0.7)
    assert res.kept == 77 and res.kept_ids == oracle.canonical_order(oracle.row_floats(x))[:77]
    res = oracle.topp_row(x, None, 1.0, 1.0)
    assert res.kept == 300


def test_two_token_closed_form():
    rng = np.random.default_rng(8)
    for _ in range(300):
        a, b = rng.standard_normal(2) * 2
        x = np.array([a, b], np.float32)
        t = oracle.to_f32(rng.uniform(0.3, 2.0))
        p = oracle.to_f32(rng.uniform(0.3, 0.99))
        d = abs(float(x[0]) - float(x[1]))
        top_prob = 1.0 / (1.0 + math.exp(-d / t))
        if abs(top_prob - p) < 1e-12:
            continue
        res = oracle.topp_row(x, None, p, t)
        assert res.kept == (1 if top_prob >= p else 2)


def test_dominant_token_keeps_one():
    # forced case of the top-p page's gate: a dominant token alone reaches any p < 1
    x = np.zeros(5000, np.float32)
    x[1234] = 80.0
    res = oracle.topp_row(x, None, oracle.to_f32(0.999999), 1.0)
    assert res.kept == 1 and res.kept_ids == [1234]


def test_huge_logits_keep_the_maximum():
    # huge finite logits (the top-p page's breakage probes): never an empty row
    x = np.array([3.0e38, 2.9e38, -3.0e38, 3.0e38], np.float32)
    res = oracle.topp_row(x, None, oracle.to_f32(0.3), 1.0)
    assert res.status == 0 and res.kept == 1 and res.kept_ids == [0]
    res = oracle.topp_row(x, None, oracle.to_f32(0.6), 1.0)
    assert res.kept == 2 and res.kept_ids == [0, 3]


def test_normaliser_matches_scipy_logsumexp():
    rng = np.random.default_rng(12)
    for _ in range(30):
        x = (rng.standard_normal(2000) * 3).astype(np.float32)
        k = int(rng.integers(1, 2000))
        t = oracle.to_f32(rng.uniform(0.5, 1.5))
        res = oracle.topp_row(x, k, oracle.to_f32(0.9), t)
        xs = np.array([res.x[i] for i in res.topk]) / t
        assert math.log(res.z) + res.m / t == pytest.approx(float(logsumexp(xs)), rel=1e-13, abs=1e-12)


def test_boundary_invariants_on_larger_rows():
    rng = np.random.default_rng(13)
    for _ in range(40):
        x = (rng.standard_normal(5000) * 2.5).astype(np.float32)
        k = int(rng.integers(1, 1025))
        p = oracle.to_f32(rng.uniform(0.5, 1.0))
        t = oracle.to_f32(rng.uniform(0.5, 1.5))
        res = oracle.topp_row(x, k, p, t)
        n = res.kept
        assert 1 <= n <= k
        assert res.kept_ids == oracle.canonical_order(res.x)[:n]
        if p < 1.0 and not res.ambiguous:
            assert math.fsum(res.weights[:n]) >= res.target
            assert n == 1 or math.fsum(res.weights[: n - 1]) < res.target


def test_neumaier_scan_reaches_with_cancellation():
    # compensation matters: 1 followed by many tiny terms
    w = [1.0] + [1e-17] * 1000
    assert oracle.neumaier_first_reach(w, 1.0 + 5e-15) == 501


def test_temperature_zero_is_greedy():
    x = np.array([0.5, 2.0, 2.0, -1.0], np.float32)
    res = oracle.topp_row(x, 3, oracle.to_f32(0.5), 0.0)
    assert res.kept == 1 and res.kept_ids == [1]


def test_minus_inf_is_masked():
    x = np.array([-np.inf, 1.0, -np.inf, 0.0], np.float32)
    res = oracle.topp_row(x, None, oracle.to_f32(0.99), 1.0)
    assert res.status == 0 and set(res.kept_ids) <= {1, 3}
    assert res.weights[2] == 0.0 and res.weights[3] == 0.0


@pytest.mark.parametrize("row,k,p,t,st", [
    ([np.nan, 1.0], None, 0.5, 1.0, 1),
    ([np.inf, 1.0], None, 0.5, 1.0, 1),
    ([-np.inf, -np.inf], None, 0.5, 1.0, 1),
    ([0.0, 1.0], 0, 0.5, 1.0, 2),
    ([0.0, 1.0], 1, 0.0, 1.0, 3),
    ([0.0, 1.0], 1, 1.5, 1.0, 3),
    ([0.0, 1.0], 1, float("nan"), 1.0, 3),
    ([0.0, 1.0], 1, 0.5, -1.0, 4),
    ([0.0, 1.0], 1, 0.5, float("inf"), 4),
    ([np.nan, 1.0], 0, 1.5, -1.0, 1),           # precedence: logits first
    ([0.0, 1.0], 0, 1.5, -1.0, 2),
])
def test_status_codes(row, k, p, t, st):
    res = oracle.topp_row(np.array(row, np.float32), k, p, t)
    assert res.status == st and res.kept == 0
