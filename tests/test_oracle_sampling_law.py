"""Pins for the oracle's Gumbel-max sampler against the categorical law (CPU only).

Gumbel-max theorem: argmax_i (x_i/T + g_i) over the kept set P is distributed as
w_i / sum_P w with w_i = exp((x_i - m)/T). Checked by chi-square (mlxcel issue #901,
"Regression guard") and by the head/tail z-tests of the vLLM PR #45996 summary ("key
source excerpts"), on a small heavy-tailed analogue of that test. Also: T = 0 returns the
canonical argmax, a one-token kept set returns that token, and the sampled support
equals the kept set.
"""
import math

import numpy as np
import pytest
from scipy.stats import chisquare

import oracle


def draw_many(x, k, p, t, n, seed0=1000, row=0):
    counts = {}
    for j in range(n):
        r = oracle.sample_row(x, k, p, t, seed0 + j, row)
        counts[r.token] = counts.get(r.token, 0) + 1
    return counts


def test_chi_square_v16_with_topk_topp():
    x = np.array([1.2, -0.3, 0.8, 0.8, 2.0, -1.0, 0.1, 0.5,
                  -2.0, 1.0, 0.0, 0.3, -0.5, 1.5, 0.7, -0.1], np.float32)
    k, p, t = 12, oracle.to_f32(0.9), oracle.to_f32(0.8)
    res = oracle.topp_row(x, k, p, t)
    kept = res.kept_ids
    n = 40000
    counts = draw_many(x, k, p, t, n)
    assert set(counts) <= set(kept)                     # support equals the kept set
    w = np.array(res.weights[: res.kept])
    probs = w / w.sum()
    obs = np.array([counts.get(i, 0) for i in kept])
    assert chisquare(obs, probs * n).pvalue > 1e-4


def test_heavy_tailed_head_and_tail_z():
    rng = np.random.default_rng(33)
    counts = rng.integers(1, 4, size=64)
    counts[0] = 500
    x = np.log(counts.astype(np.float64)).astype(np.float32)
    n = 30000
    got = draw_many(x, None, 1.0, 1.0, n, seed0=77)
    total = counts.sum()
    p0 = counts[0] / total
    obs0 = got.get(0, 0)
    z0 = (obs0 - p0 * n) / math.sqrt(n * p0 * (1 - p0))
    tail = n - obs0
    zt = (tail - (1 - p0) * n) / math.sqrt(n * p0 * (1 - p0))
    assert abs(z0) < 5 and abs(zt) < 5


def test_temperature_zero_and_single_token():
    x = np.array([0.1, 3.0, 3.0, -2.0], np.float32)
    assert oracle.sample_row(x, None, 1.0, 0.0, 5, 0).token == 1
    # k = 1 leaves one token: noise cannot change it
    for s in range(50):
        assert oracle.sample_row(x, 1, 1.0, 1.0, s, 3).token == 1


def test_masked_tokens_never_sampled():
    x = np.array([-np.inf, 0.0, -np.inf, 0.0], np.float32)
    got = draw_many(x, None, 1.0, 1.0, 400)
    assert set(got) == {1, 3}


def test_same_seed_same_stream_and_row_dependence():
    x = np.zeros(64, np.float32)
    a = [oracle.sample_row(x, None, 1.0, 1.0, 42, r).token for r in range(20)]
    b = [oracle.sample_row(x, None, 1.0, 1.0, 42, r).token for r in range(20)]
    assert a == b and len(set(a)) > 5


def test_gap_reports_near_ties():
    x = np.zeros(4, np.float32)
    r = oracle.sample_row(x, None, 1.0, 1.0, 3, 0)
    assert r.gap > 0 and math.isfinite(r.gap)
    r = oracle.sample_row(x, 1, 1.0, 1.0, 3, 0)
    assert r.gap == math.inf
