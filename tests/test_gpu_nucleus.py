"""Rows with top-k off and top-p or min-p on, called without a top-k array, take the nucleus
pass (rows x chunks workgroups weigh the row into per-bin histograms; the row kernel resolves
only the bin where the nucleus ends). It must give the same bytes as the single-workgroup
row-streaming path (forced with TS_KNOB_FORCE_EXACT) - kept counts, masks, tokens and
logprobs - and match the oracle on sampled rows. Covers spread rows, bf16-rounded ties, a
narrow near-uniform row, min-p with and without top-p, and an all-equal row whose cut bin
exceeds LDS (the row-streaming fallback).
"""
import numpy as np
import pytest

import oracle
import top_select_gumbel_amd as ts
from top_select_gumbel_amd import workloads as wl
from gpu_helpers import banner, check_samples, check_topp, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _torch():
    return torch_cuda()


def d(a, dt):
    return None if a is None else dev(np.asarray(a, dt))


def both(fn):
    """fn() with the nucleus passes (forced for every call size) and with the row-streaming
    path; a third run with the default routing (small sampling calls take the split nucleus)
    must give the same bytes as the first."""
    torch = torch_cuda()
    out = []
    for exact, passes in ((0, 1), (1, 1), (0, 0)):
        old = ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, exact)
        oldp = ts.ts_debug_set(ts.TS_KNOB_NUCLEUS_PASSES, passes)
        try:
            res = fn()
            torch.cuda.synchronize()
            out.append([None if v is None else host(v) for v in res])
        finally:
            ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, old)
            ts.ts_debug_set(ts.TS_KNOB_NUCLEUS_PASSES, oldp)
    for a, b in zip(out[0], out[2]):
        assert (a is None and b is None) or np.array_equal(a, b), "default routing differs from the nucleus passes"
    return out[:2]


def mixed_rows(seed, rows, vocab):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, vocab)) * 2.5
    x[1] = np.round(rng.standard_normal(vocab) * 1e5 / 1024) * 1024          # bf16-like ties
    x[2] = 1.0 + 1e-6 * rng.standard_normal(vocab)                           # narrow
    x[3, rng.choice(vocab, vocab // 3, replace=False)] = -np.inf             # masked tokens
    x[4] = np.round(rng.standard_normal(vocab), 1)                           # heavy ties
    x = x.astype(np.float32)
    p = rng.uniform(0.3, 0.99, rows).astype(np.float32)
    p[5] = 1.0                                                                # min-p only rows below
    t = rng.uniform(0.5, 1.5, rows).astype(np.float32)
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    return x, p, t, seeds


@pytest.mark.parametrize("vocab", [151936, 40000])
def test_nucleus_matches_row_streaming_and_oracle(vocab):
    x, p, t, seeds = mixed_rows(71, 12, vocab)
    banner(f"nucleus top-p rows 12x{vocab}")
    (k1, m1, s1), (k2, m2, s2) = both(lambda: ts.ts_topp_mask(dev(x), None, d(p, np.float32), d(t, np.float32)))
    assert np.array_equal(s1, s2) and np.array_equal(k1, k2) and np.array_equal(m1, m2)
    sd = dev(seeds)
    (a1, u1), (a2, u2) = both(lambda: ts.ts_sample_rows(dev(x), None, d(p, np.float32), d(t, np.float32), sd))
    assert np.array_equal(a1, a2) and np.array_equal(u1, u2)
    rows = [0, 1, 2, 3, 4, 5]
    check_topp(x[rows], None, p[rows], t[rows], k1[rows], m1[rows], s1[rows], "nucleus")
    check_samples(x[rows], None, p[rows], t[rows], seeds[rows], a1[rows], u1[rows], k1[rows], "nucleus",
                  row_ids=rows)


def test_nucleus_minp_and_logp():
    x, p, t, seeds = mixed_rows(72, 10, 60000)
    mp = np.linspace(0.0, 0.3, 10).astype(np.float32)
    banner("nucleus min-p rows 10x60000")
    (k1, m1, s1), (k2, m2, s2) = both(lambda: ts.ts_topp_mask_minp(dev(x), None, d(p, np.float32),
                                                                   d(t, np.float32), d(mp, np.float32)))
    assert np.array_equal(s1, s2) and np.array_equal(k1, k2) and np.array_equal(m1, m2)
    sd = dev(seeds)
    (a1, u1), (a2, u2) = both(lambda: ts.ts_sample_rows_minp(dev(x), None, d(p, np.float32), d(t, np.float32),
                                                              d(mp, np.float32), sd))
    assert np.array_equal(a1, a2) and np.array_equal(u1, u2)
    for r in (0, 3, 6, 9):
        o = oracle.sample_minp_row(x[r], None, oracle.to_f32(p[r]), oracle.to_f32(t[r]), oracle.to_f32(mp[r]),
                                   int(seeds[r]), r)
        assert s1[r] == o.status
        if o.topp.minp_ambiguous or o.topp.ambiguous:
            continue
        assert k1[r] == o.topp.kept
        if o.gap >= 1e-4:
            assert a1[r] == o.token
    (b1, l1, e1, v1), (b2, l2, e2, v2) = both(lambda: ts.ts_sample_rows_logp(dev(x), None, d(p, np.float32),
                                                                             d(t, np.float32), sd))
    assert np.array_equal(b1, b2) and np.array_equal(l1, l2) and np.array_equal(e1, e2)


def test_nucleus_decode_rows_without_topk_array():
    b = wl.decode_topp_only()
    banner("nucleus decode rows 64x151936, top_k NULL")
    sd = dev(b.seeds)
    (a1, u1), (a2, u2) = both(lambda: ts.ts_sample_rows(dev(b.logits), None, d(b.p, np.float32),
                                                        d(b.t, np.float32), sd))
    assert np.array_equal(a1, a2) and (u1 == 0).all()
    (k1, _, _), (k2, _, _) = both(lambda: ts.ts_topp_mask(dev(b.logits), None, d(b.p, np.float32),
                                                         d(b.t, np.float32), want_mask=False))
    assert np.array_equal(k1, k2)


def test_nucleus_cut_bin_larger_than_lds_falls_back():
    x = np.full((3, 30000), 2.5, np.float32)          # all equal: one bin of 30000 tokens
    x[1, ::7] = 3.0
    p = np.array([0.5, 0.9, 0.31], np.float32)
    t = np.ones(3, np.float32)
    seeds = np.arange(3, dtype=np.uint64) + 5
    banner("nucleus all-equal rows 3x30000 (fallback)")
    (k1, m1, _), (k2, m2, _) = both(lambda: ts.ts_topp_mask(dev(x), None, d(p, np.float32), d(t, np.float32)))
    assert np.array_equal(k1, k2) and np.array_equal(m1, m2)
    (a1, _), (a2, _) = both(lambda: ts.ts_sample_rows(dev(x), None, d(p, np.float32), d(t, np.float32), dev(seeds)))
    assert np.array_equal(a1, a2)
    check_topp(x, None, p, t, k1, m1, np.zeros(3, np.int32), "all-equal")
