"""Pins of the oracle's temperature-scaled log-sum-exp and selected-token logprob.

[LOGP] "Design: the numeric contract" defines lse = m + log(sum exp(z - m)) and
logp = min(z_t - lse, 0), temperature applied in the epilogue. The pins are closed forms
(all-equal rows, two-token rows), scipy's logsumexp, the normalisation of the distribution
the logprobs describe, masked (-inf) tokens, and exact temperature scaling.
"""
import math

import numpy as np
import pytest

import oracle


def test_all_equal_row_closed_form():
    for v, c, t in ((16, 0.0, 1.0), (1000, 3.25, 0.5), (7, -2.0, 1.75)):
        row = np.full(v, c, np.float32)
        lse, logp = oracle.lse_logp_row(row, t, 3)
        assert lse == pytest.approx(c / t + math.log(v), abs=1e-12)
        assert logp == pytest.approx(-math.log(v), abs=1e-12)


def test_two_tokens_closed_form():
    for a, b, t in ((1.0, 0.0, 1.0), (0.0, 4.0, 0.5), (-3.5, 2.25, 2.0)):
        row = np.array([a, b], np.float32)
        hi, lo = max(a, b), min(a, b)
        want = hi / t + math.log1p(math.exp(-(hi - lo) / t))
        lse0, lp0 = oracle.lse_logp_row(row, t, 0)
        lse1, lp1 = oracle.lse_logp_row(row, t, 1)
        assert lse0 == pytest.approx(want, abs=1e-12) and lse1 == lse0
        # p0 = 1 / (1 + exp((b - a) / t))
        assert lp0 == pytest.approx(-math.log1p(math.exp((b - a) / t)), abs=1e-12)
        assert lp1 == pytest.approx(-math.log1p(math.exp((a - b) / t)), abs=1e-12)


def test_matches_scipy_logsumexp():
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(5)
    for _ in range(20):
        v = int(rng.integers(2, 3000))
        t = float(np.float32(rng.uniform(0.2, 3.0)))
        row = (rng.standard_normal(v) * rng.uniform(0.5, 20)).astype(np.float32)
        tok = int(rng.integers(0, v))
        lse, logp = oracle.lse_logp_row(row, t, tok)
        want = float(special.logsumexp(row.astype(np.float64) / t))
        assert lse == pytest.approx(want, rel=1e-13, abs=1e-12)
        assert logp == pytest.approx(min(float(row[tok]) / t - want, 0.0), rel=1e-12, abs=1e-12)


def test_logprobs_normalise_and_are_nonpositive():
    rng = np.random.default_rng(6)
    for t in (0.3, 1.0, 2.5):
        row = (rng.standard_normal(40) * 3).astype(np.float32)
        lps = [oracle.lse_logp_row(row, t, i)[1] for i in range(40)]
        assert max(lps) <= 0.0
        assert math.fsum(math.exp(lp) for lp in lps) == pytest.approx(1.0, abs=1e-12)
        # the order of the logprobs is the order of the logits
        assert np.argmax(lps) == int(np.argmax(row))


def test_masked_tokens_and_greedy():
    row = np.array([0.5, -np.inf, -np.inf, 0.5], np.float32)
    lse, logp = oracle.lse_logp_row(row, 1.0, 0)
    assert lse == pytest.approx(0.5 + math.log(2.0), abs=1e-12)
    assert logp == pytest.approx(-math.log(2.0), abs=1e-12)
    assert oracle.lse_logp_row(row, 1.0, 1)[1] == -math.inf
    assert oracle.lse_logp_row(row, 0.0, 0) == (math.inf, 0.0)


def test_temperature_scales_exactly():
    # x / T with T a power of two is exact, so lse(x, T) must equal lse(x / T, 1)
    rng = np.random.default_rng(7)
    row = (rng.standard_normal(500) * 4).astype(np.float32)
    for t in (0.25, 2.0, 8.0):
        a = oracle.lse_logp_row(row, t, 17)
        b = oracle.lse_logp_row((row / np.float32(t)).astype(np.float32), 1.0, 17)
        assert a[0] == pytest.approx(b[0], abs=1e-12) and a[1] == pytest.approx(b[1], abs=1e-12)


def test_batched_form_rejects_rows():
    x = np.zeros((3, 8), np.float32)
    x[1, 2] = np.nan
    out = oracle.sample_logp_rows(x, np.array([8, 8, 8]), np.ones(3, np.float32), np.ones(3, np.float32),
                                  np.array([1, 2, 3], np.uint64))
    assert out[0][0].status == 0 and out[0][1] == pytest.approx(math.log(8.0))
    assert out[1][0].status != 0 and math.isnan(out[1][1]) and math.isnan(out[1][2])
