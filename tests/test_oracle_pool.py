"""The row-parallel checker itself (CPU only): it passes the oracle's own outputs and
catches a planted mistake in each kind of output."""
import numpy as np
import pytest

import oracle
import oracle_pool as op


def small():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((6, 3000)) * 2).astype(np.float32)
    x[5] = 1.5                                   # all equal
    k = np.array([5, 100, 3000, 1, 64, 40], np.int32)
    p = np.array([0.9, 0.7, 0.95, 1.0, 0.5, 0.8], np.float32)
    t = np.array([1.0, 0.8, 1.2, 1.0, 0.6, 1.0], np.float32)
    seeds = rng.integers(0, 2 ** 64, 6, dtype=np.uint64)
    return x, k, p, t, seeds


def test_pool_checks_accept_the_oracle_and_catch_planted_mistakes():
    x, k, p, t, seeds = small()
    st, idx = oracle.topk_select(x, k, 100)
    op.check_topk(x, k, 100, idx, st, "ok")
    bad = idx.copy()
    bad[1, 3] += 1
    with pytest.raises(AssertionError):
        op.check_topk(x, k, 100, bad, st, "planted")
    res = oracle.topp_mask(x, k, p, t)
    kept = np.array([r.kept for r in res], np.int32)
    mask = np.zeros(x.shape, np.uint8)
    for r, o in enumerate(res):
        mask[r, o.kept_ids] = 1
    stp = np.array([r.status for r in res], np.int32)
    assert op.check_topp(x, k, p, t, kept, mask, stp, "ok") == []
    mask[1, res[1].order[res[1].kept]] = 1       # one token past the prefix
    with pytest.raises(AssertionError):
        op.check_topp(x, k, p, t, kept, mask, stp, "planted")
    sr = oracle.sample_rows(x, k, p, t, seeds)
    tok = np.array([r.token for r in sr], np.int32)
    sts = np.array([r.status for r in sr], np.int32)
    op.check_samples(x, k, p, t, seeds, tok, sts, kept, "ok")
    tok2 = tok.copy()
    j = next(r for r, o in enumerate(sr) if o.topp.kept > 1 and o.gap >= 1e-4)
    tok2[j] = [i for i in sr[j].topp.kept_ids if i != tok[j]][0]
    with pytest.raises(AssertionError):
        op.check_samples(x, k, p, t, seeds, tok2, sts, kept, "planted")
