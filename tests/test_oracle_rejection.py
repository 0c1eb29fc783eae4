"""Pins for the oracle's dual-pivot rejection sampler (CPU only).

mlxcel issue #901, "Regression guard": the sampled support must equal the filters' set
(with the token-id tie rule) and the frequencies inside it must follow the renormalised
truncated distribution (chi-square); same seed, same stream; the cap's fallback draws
valid samples. The support is computed here from its definition with a stable argsort
and exact rational sums of binary64 weights (not with the oracle's integer masses), and
the law from math.exp. Closed forms: two tokens, all-equal rows, a dominant token,
k = 1, T = 0, and a case where the joint filter (both tests against the full
distribution) and top-p over the top-k set differ.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.stats import chisquare

import oracle
from oracle.rejection import rejection_sample_row

F32 = oracle.to_f32


def support_by_definition(x, k, p, t, min_p):
    """Canonical prefix: top-k, top-p against the whole row, min-p; exact rationals."""
    x = np.asarray(x, np.float32).astype(np.float64)
    V = len(x)
    order = list(np.argsort(-x, kind="stable"))
    m = x[order[0]]
    w = [math.exp((x[i] - m) / t) for i in order]
    n_k = V if k is None else min(k, V)
    n_p = V
    if p != 1.0:
        z = sum(Fraction(v) for v in w)
        target = Fraction(p) * z
        acc = Fraction(0)
        for n, v in enumerate(w, start=1):
            acc += Fraction(v)
            if acc >= target:
                n_p = n
                break
    n_m = sum(1 for v in w if v >= min_p) if min_p else V
    n = min(n_k, n_p, n_m)
    return [int(i) for i in order[:n]], [w[j] for j in range(n)]


def draws(x, k, p, t, min_p, n, max_rounds=32, seed0=5000, row=0):
    out = []
    for s in range(n):
        r = rejection_sample_row(x, k, p, t, min_p, seed0 + s, row, max_rounds)
        assert r.status == oracle.STATUS_OK
        out.append((r.token, r.rounds))
    return out


def law_check(x, k, p, t, min_p, n, max_rounds=32):
    sup, w = support_by_definition(x, k, p, t, min_p)
    got = draws(x, k, p, t, min_p, n, max_rounds)
    toks = [g for g, _ in got]
    assert set(toks) <= set(sup)
    obs = np.array([toks.count(i) for i in sup], float)
    probs = np.array(w) / sum(w)
    assert chisquare(obs, probs * n).pvalue > 1e-4
    return got


X16 = np.array([1.2, -0.3, 0.8, 0.8, 2.0, -1.0, 0.1, 0.5,
                -2.0, 1.0, 0.0, 0.3, -0.5, 1.5, 0.7, -0.1], np.float32)


def test_law_topk():
    got = law_check(X16, 6, 1.0, F32(0.8), 0.0, 12000)
    assert max(r for _, r in got) > 1          # rejections happen


def test_law_topp_whole_row():
    law_check(X16, None, F32(0.7), F32(1.3), 0.0, 12000)


def test_law_joint_with_minp():
    law_check(X16, 10, F32(0.9), F32(0.6), F32(0.05), 12000)


def test_law_of_the_fallback():
    got = law_check(X16, 5, F32(0.8), F32(1.0), 0.0, 8000, max_rounds=0)
    assert all(r == -1 for _, r in got)
    got = law_check(X16, 3, 1.0, F32(1.0), 0.0, 8000, max_rounds=1)   # mixed: accepted or fallback
    assert {r for _, r in got} == {1, -1}


def test_support_random_tiny_rows_with_ties():
    rng = np.random.default_rng(12)
    for case in range(150):
        V = int(rng.integers(1, 13))
        if case % 2:
            x = rng.integers(-2, 3, size=V).astype(np.float32)
        else:
            x = rng.standard_normal(V).astype(np.float32)
        k = int(rng.integers(1, V + 2))
        p = F32(rng.uniform(0.05, 1.0)) if case % 3 else 1.0
        t = F32(rng.uniform(0.3, 2.0))
        mp = F32(rng.uniform(0.0, 0.5)) if case % 4 == 0 else 0.0
        sup, _ = support_by_definition(x, k, p, t, mp)
        for s in range(12):
            r = rejection_sample_row(x, k, p, t, mp, 100 * case + s, case)
            if r.ambiguous:
                continue
            assert r.support_n == len(sup)
            assert r.token in sup


def test_two_token_closed_form():
    d, t = 1.3, 0.7
    x = np.array([0.0, d], np.float32)
    n = 20000
    got = [g for g, _ in draws(x, None, 1.0, F32(t), 0.0, n)]
    p1 = 1.0 / (1.0 + math.exp(-float(np.float32(d)) / F32(t)))
    z = (got.count(1) - n * p1) / math.sqrt(n * p1 * (1 - p1))
    assert abs(z) < 5


def test_all_equal_row_keeps_lowest_ids():
    x = np.full(40, 2.5, np.float32)
    got = [g for g, _ in draws(x, 7, 1.0, 1.0, 0.0, 7000)]
    assert set(got) == set(range(7))
    assert chisquare(np.bincount(got, minlength=7)).pvalue > 1e-4
    # p = 0.5 over 8 equal weights: the mass of 4 tokens equals the target exactly, so the
    # nucleus is {0..3} and a candidate whose mass above equals the target is rejected.
    got = [g for g, _ in draws(np.ones(8, np.float32), None, 0.5, 1.0, 0.0, 800)]
    assert set(got) == {0, 1, 2, 3}


def test_degenerate_cases():
    x = np.array([0.1, 3.0, 3.0, -2.0], np.float32)
    r = rejection_sample_row(x, None, 1.0, 0.0, 0.0, 9, 0)
    assert (r.token, r.rounds) == (1, 0)                       # T = 0: greedy
    for s in range(40):
        assert rejection_sample_row(x, 1, 1.0, 1.0, 0.0, s, 2).token == 1       # k = 1
    y = np.array([0.0, 0.0, 40.0, 0.0, 0.0], np.float32)
    for s in range(40):
        assert rejection_sample_row(y, None, F32(0.5), 1.0, 0.0, s, 1).token == 2   # dominant
        assert rejection_sample_row(y, None, 1.0, 1.0, F32(0.3), s, 1).token == 2   # min-p
    m = np.array([-np.inf, 0.0, -np.inf, 0.0], np.float32)
    assert {rejection_sample_row(m, None, 1.0, 1.0, 0.0, s, 0).token for s in range(200)} == {1, 3}


def test_joint_filter_differs_from_topp_over_topk():
    # weights 1, 0.4, 0.4, 0.2: top-p 0.65 over the whole row keeps 2 tokens (1.4 / 2.0 =
    # 0.7), so the joint support with k = 2 has 2 tokens; top-p over the top-k set would
    # keep one (1.0 / 1.4 >= 0.65).
    x = np.log(np.array([1.0, 0.4, 0.4, 0.2])).astype(np.float32)
    p = F32(0.65)
    r = rejection_sample_row(x, 2, p, 1.0, 0.0, 1, 0)
    assert r.support_n == 2
    assert oracle.topp_row(x, 2, p, 1.0).kept == 1
    got = [g for g, _ in draws(x, 2, p, 1.0, 0.0, 6000)]
    assert set(got) == {0, 1}
    p0 = 1.0 / 1.4
    z = (got.count(0) - 6000 * p0) / math.sqrt(6000 * p0 * (1 - p0))
    assert abs(z) < 5


def test_status_codes_and_precedence():
    x = np.zeros(8, np.float32)
    bad = x.copy()
    bad[3] = np.nan
    assert rejection_sample_row(bad, 0, 2.0, -1.0, 3.0, 1, 0).status == oracle.STATUS_NONFINITE
    assert rejection_sample_row(x, 0, 2.0, -1.0, 3.0, 1, 0).status == oracle.STATUS_BAD_K
    assert rejection_sample_row(x, 3, 0.0, -1.0, 3.0, 1, 0).status == oracle.STATUS_BAD_P
    assert rejection_sample_row(x, 3, 0.5, -1.0, 3.0, 1, 0).status == oracle.STATUS_BAD_T
    assert rejection_sample_row(x, 3, 0.5, 1.0, 3.0, 1, 0).status == oracle.STATUS_BAD_MINP
    assert rejection_sample_row(np.full(4, -np.inf, np.float32), None, 1.0, 1.0, 0.0, 1, 0).status \
        == oracle.STATUS_NONFINITE


def test_same_seed_same_stream_and_rows_differ():
    x = np.zeros(64, np.float32)
    a = [rejection_sample_row(x, 32, 1.0, 1.0, 0.0, 42, r).token for r in range(20)]
    b = [rejection_sample_row(x, 32, 1.0, 1.0, 0.0, 42, r).token for r in range(20)]
    assert a == b and len(set(a)) > 5


@pytest.mark.slow
def test_near_uniform_long_row_converges():
    rng = np.random.default_rng(7)
    x = (1.0 + 1e-6 * rng.standard_normal(152000)).astype(np.float32)
    sup, _ = support_by_definition(x, 2048, 1.0, 1.0, 0.0)
    for s in range(3):
        r = rejection_sample_row(x, 2048, 1.0, 1.0, 0.0, s, 0)
        assert 1 <= r.rounds <= 32
        assert r.token in set(sup)


def test_worked_trajectory_with_injected_words():
    # x = 0..15, T = 1, k = 4, weights w_i = e^(i - 15), worked by hand from the page's rule
    # (second pivot halfway between the candidate's probability and the upper bound, which
    # starts at the maximum's weight 1). Round 0 draws token 9: 6 tokens rank above it
    # (reject); pivot (e^-6 + 1) / 2 = 0.5012 has only token 15 above it (< k), so the support
    # lies above the candidate: eligible {10..15}, upper bound 0.5012. Round 1, word 0: the
    # first eligible token, 10: 5 above (reject); pivot (e^-5 + 0.5012) / 2 = 0.2540 has 2
    # above (15, 14): eligible {11..15}, bound 0.2540. Round 2: token 11, 4 above (reject);
    # pivot (e^-4 + 0.2540) / 2 = 0.1362 still has 2 above (e^-2 = 0.1353 is below it):
    # eligible {12..15}. Round 3: token 12, 3 above: accepted at round 4. (A midpoint taken
    # on logits, (9 + 15) / 2 = 12, would have accepted at round 3.)
    x = np.arange(16, dtype=np.float32)
    e = [math.exp(i - 15) for i in range(16)]
    w0 = int((sum(e[:9]) + 0.5 * e[9]) / sum(e) * 2 ** 32)
    r = rejection_sample_row(x, 4, 1.0, 1.0, 0.0, 0, 0, words=lambda j: w0 if j == 0 else 0)
    assert (r.token, r.rounds, r.ambiguous) == (12, 4, False)
    # The other branch: T = 10, weights e^((i - 15) / 10), words all 0 (each round draws the
    # lowest eligible id). Round 0: token 0 (weight e^-1.5 = 0.2231), 15 above (reject);
    # pivot (0.2231 + 1) / 2 = 0.6116 has 5 above it (15..11; e^-0.5 = 0.6065 is below), >= k,
    # so the support lies above the second pivot: eligible {11..15}, the bound stays 1.
    # Round 1: token 11, 4 above (reject); pivot (e^-0.4 + 1) / 2 = 0.8352 has 2 above
    # (15, 14): eligible {12..15}, bound 0.8352. Round 2: token 12, 3 above: accepted.
    r = rejection_sample_row(x, 4, 1.0, F32(10.0), 0.0, 0, 0, words=lambda j: 0)
    assert (r.token, r.rounds, r.ambiguous) == (12, 3, False)
    # Top-p form of the T = 1 walk: p such that the target lies between the masses of
    # {12..15} and {11..15}: the support is {11..15} (5 tokens); round 0 draws 9 (rejected:
    # mass above it exceeds the target), pivot 0.5012 has only token 15 above it, whose mass
    # is below the target, so eligible {10..15}, bound 0.5012; word 0 draws 10 (mass above
    # it reaches the target: rejected); pivot 0.2540 has {15, 14} above it, mass below the
    # target: eligible {11..15}; word 0 draws 11, whose mass above is below the target:
    # accepted at round 3.
    above = lambda n: sum(e[16 - n:]) / sum(e)          # mass of the top n tokens
    p = F32(0.5 * (above(4) + above(5)))
    r = rejection_sample_row(x, None, p, 1.0, 0.0, 0, 0, words=lambda j: w0 if j == 0 else 0)
    assert (r.token, r.rounds, r.support_n, r.support_exact) == (11, 3, 5, True)


def test_pivot_ties_flag_the_row():
    # Weights 1, 0.6, 0.2, 0.2 with k = 2: the injected word draws token 2 (mid-way through
    # its mass); the second pivot (0.2 + 1) / 2 = 0.6 equals token 1's weight, which a GPU
    # weight 1.6e-7 off could put on either side, so the row is flagged (validity only). With
    # 0.59 in place of 0.6 the pivot is clear of every weight and the row is not flagged.
    def run(w1):
        x = np.log(np.array([1.0, w1, 0.2, 0.2])).astype(np.float32)
        w = np.exp(x.astype(np.float64) - float(x.max()))
        M = np.floor(np.ldexp(w, 63 - 3))
        word = int((M[0] + M[1] + 0.5 * M[2]) / M.sum() * 2 ** 32)
        return rejection_sample_row(x, 2, 1.0, 1.0, 0.0, 0, 0, words=lambda j: word if j == 0 else 0)
    r = run(0.6)
    assert r.ambiguous and r.token in (0, 1)
    r = run(0.59)
    assert not r.ambiguous and r.token in (0, 1)
