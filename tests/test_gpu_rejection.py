"""GPU parity of ts_sample_rows_rejection (dual-pivot rejection sampling) against the oracle.

mlxcel issue #901, "Regression guard". Both sides run the same rounds on the same Philox
words, with integer masses; the GPU's weights are fp32-accurate, so the oracle flags rows
where a CDF crossing, a top-p test or a min-p test lies within that error of flipping.
Unflagged rows: the token and the round count equal the oracle's. Flagged rows: the token
lies in the support: its rank is below n_S, and below k always (the k boundary is an exact
count); only where the top-p or min-p test at the support's edge is within the weight error
may the GPU's support run up to 3 tokens longer. Also: the law of the draws (chi-square
against the renormalised truncated distribution), the forced fallback, status codes and
poisoned outputs, misaligned rows, and every row of the decode shapes.
"""
import math

import numpy as np
import pytest
from scipy.stats import chisquare

import oracle
import top_select_gumbel_amd as ts
from top_select_gumbel_amd import workloads as wl
from gpu_helpers import banner, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _torch():
    return torch_cuda()


def d(a, dt):
    return None if a is None else dev(np.asarray(a, dt))


def run(x, k, p, t, mp, seeds, max_rounds=32, x_dev=None):
    torch = torch_cuda()
    tok, rnd, st = ts.ts_sample_rows_rejection(dev(x) if x_dev is None else x_dev, d(k, np.int32),
                                               d(p, np.float32), d(t, np.float32), d(mp, np.float32),
                                               dev(np.asarray(seeds, np.uint64)), max_rounds)
    torch.cuda.synchronize()
    return host(tok), host(rnd), host(st)


def check(x, k, p, t, mp, seeds, tok, rnd, st, label, max_rounds=32, rows=None):
    rows = range(x.shape[0]) if rows is None else rows
    flagged = 0
    for r in rows:
        o = oracle.rejection_sample_row(x[r], None if k is None else int(k[r]),
                                        None if p is None else oracle.to_f32(p[r]),
                                        None if t is None else oracle.to_f32(t[r]),
                                        None if mp is None else oracle.to_f32(mp[r]),
                                        int(seeds[r]), r, max_rounds)
        assert st[r] == o.status, f"{label} row {r}: status {st[r]} vs {o.status}"
        if o.status != 0:
            assert tok[r] == -1 and rnd[r] == 0, f"{label} row {r}: poisoned outputs {tok[r]} {rnd[r]}"
            continue
        if o.ambiguous:
            flagged += 1
            rank = int(np.nonzero(o.order == tok[r])[0][0])
            k_eff = x.shape[1] if k is None else min(int(k[r]), x.shape[1])
            bound = o.support_n if o.support_exact else min(k_eff, o.support_n + 3)
            assert rank < bound, \
                f"{label} row {r}: token rank {rank}, support {o.support_n} (exact {o.support_exact}), k {k_eff}"
            continue
        assert (tok[r], rnd[r]) == (o.token, o.rounds), \
            f"{label} row {r}: gpu (token {tok[r]}, round {rnd[r]}) vs oracle ({o.token}, {o.rounds})"
    return flagged


@pytest.mark.parametrize("seed,vocab,ties,masked", [(21, 1000, 0, 0.0), (22, 5000, 0, 0.05),
                                                    (23, 3000, 4, 0.0), (24, 2049, 2, 0.2)])
def test_parity_mixed_rows(seed, vocab, ties, masked):
    b = wl.rejection_mix(seed, 96, vocab, tie_levels=ties, masked=masked)
    banner(f"rejection parity seed={seed} {b.logits.shape} ties={ties} masked={masked}")
    tok, rnd, st = run(b.logits, b.k, b.p, b.t, b.min_p, b.seeds)
    flagged = check(b.logits, b.k, b.p, b.t, b.min_p, b.seeds, tok, rnd, st, b.name)
    assert flagged <= 5
    assert (rnd > 1).any()                           # some rows needed more than one round


@pytest.mark.parametrize("max_rounds", [0, 1, 2])
def test_forced_fallback(max_rounds):
    b = wl.rejection_mix(31 + max_rounds, 64, 4000)
    banner(f"rejection fallback max_rounds={max_rounds}")
    tok, rnd, st = run(b.logits, b.k, b.p, b.t, b.min_p, b.seeds, max_rounds=max_rounds)
    check(b.logits, b.k, b.p, b.t, b.min_p, b.seeds, tok, rnd, st, f"fallback{max_rounds}", max_rounds)
    live = (st == 0) & (b.t != 0)
    if max_rounds == 0:
        assert (rnd[live] == -1).all()
    else:
        assert (rnd[live] == -1).any()


def test_misaligned_rows_and_ragged_tail():
    torch = torch_cuda()
    b = wl.rejection_mix(41, 40, 1003)
    banner("rejection misaligned stride 1005")
    full = np.zeros((40, 1005), np.float32)
    full[:, :1003] = b.logits
    xd = dev(full)[:, :1003]
    assert xd.stride(0) == 1005
    tok, rnd, st = run(b.logits, b.k, b.p, b.t, b.min_p, b.seeds, x_dev=xd)
    check(b.logits, b.k, b.p, b.t, b.min_p, b.seeds, tok, rnd, st, "misaligned")


def test_status_codes_and_greedy():
    x = np.random.default_rng(5).standard_normal((7, 300)).astype(np.float32)
    x[0, 17] = np.nan
    x[1, 3] = np.inf
    x[2, :] = -np.inf
    k = np.array([5, 5, 5, 0, 5, 5, 5], np.int32)
    p = np.array([0.9, 0.9, 0.9, 0.9, 0.0, 0.9, 0.9], np.float32)
    t = np.array([1, 1, 1, 1, 1, -1, 0], np.float32)
    mp = np.zeros(7, np.float32)
    seeds = np.arange(7, dtype=np.uint64)
    banner("rejection status codes")
    tok, rnd, st = run(x, k, p, t, mp, seeds)
    assert st.tolist() == [1, 1, 1, 2, 3, 4, 0]
    assert tok[:6].tolist() == [-1] * 6
    assert tok[6] == int(np.argmax(x[6])) and rnd[6] == 0
    mp2 = np.full(7, 1.5, np.float32)
    x2 = np.zeros((7, 300), np.float32)
    _, _, st2 = run(x2, np.full(7, 5, np.int32), np.full(7, 0.9, np.float32), np.ones(7, np.float32), mp2, seeds)
    assert (st2 == 5).all()
    with pytest.raises(ts.TopSelectError):
        run(x2, None, None, None, None, seeds, max_rounds=65)


def test_law_chi_square_many_rows():
    torch = torch_cuda()
    xr = np.array([1.2, -0.3, 0.8, 0.8, 2.0, -1.0, 0.1, 0.5,
                   -2.0, 1.0, 0.0, 0.3, -0.5, 1.5, 0.7, -0.1], np.float32)
    rows, launches = 4096, 64
    x = dev(np.tile(xr, (rows, 1)))
    cases = [(6, 1.0, 0.8, 0.0), (16, 0.7, 1.3, 0.0), (10, 0.9, 0.6, 0.05)]
    for kk, pp, tt, mm in cases:
        banner(f"rejection law k={kk} p={pp} T={tt} min_p={mm}")
        k = d(np.full(rows, kk), np.int32)
        p = d(np.full(rows, pp), np.float32)
        t = d(np.full(rows, tt), np.float32)
        mp = d(np.full(rows, mm), np.float32)
        counts = np.zeros(16, np.int64)
        for j in range(launches):
            seeds = dev(np.full(rows, 0xABC00000 + j, np.uint64))
            tok, _, st = ts.ts_sample_rows_rejection(x, k, p, t, mp, seeds)
            counts += np.bincount(host(tok), minlength=16)
        torch.cuda.synchronize()
        o = oracle.rejection_sample_row(xr, kk, oracle.to_f32(pp), oracle.to_f32(tt), oracle.to_f32(mm), 1, 0)
        sup = [int(i) for i in o.order[: o.support_n]]
        assert counts[[i for i in range(16) if i not in sup]].sum() == 0
        m = float(xr.max())
        w = np.array([math.exp((float(xr[i]) - m) / oracle.to_f32(tt)) for i in sup])
        n = counts.sum()
        assert chisquare(counts[sup], w / w.sum() * n).pvalue > 1e-4


def test_decode_shape_every_row():
    b = wl.decode()
    banner(f"rejection decode shape {b.logits.shape}")
    tok, rnd, st = run(b.logits, b.k, b.p, b.t, None, b.seeds)
    assert (st == 0).all()
    check(b.logits, b.k, b.p, b.t, None, b.seeds, tok, rnd, st, "decode")
    top = wl.decode_topp_only()
    tok, rnd, st = run(top.logits, top.k, top.p, top.t, None, top.seeds)
    check(top.logits, top.k, top.p, top.t, None, top.seeds, tok, rnd, st, "decode_topp_only")


def test_near_uniform_long_row():
    b = wl.indexer_near_uniform()
    x = np.repeat(b.logits, 4, axis=0)
    seeds = np.arange(4, dtype=np.uint64) + 99
    banner("rejection near-uniform 152000, k = 2048")
    tok, rnd, st = run(x, np.full(4, 2048, np.int32), None, np.ones(4, np.float32), None, seeds)
    check(x, np.full(4, 2048, np.int32), None, np.ones(4, np.float32), None, seeds, tok, rnd, st, "near_uniform")
    assert (rnd >= 1).all() and (rnd <= 32).all()
