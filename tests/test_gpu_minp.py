"""GPU parity of the min-p entry points (ts_topp_mask_minp, ts_sample_rows_minp) against the
binary64 oracle, through the C ABI.

Matching rules as for top-p: kept counts equal the oracle's except on rows whose top-p or
min-p boundary the oracle flags as ambiguous (a weight within 1e-6 of min_p, or an
uncertified top-p boundary), where they may differ by at most 3; the kept set is the
canonical prefix; sampled ids equal the oracle's argmax over the GPU's kept set unless its
top-two gap is below 1e-4. min_p = 0 gives the bytes of the entry points without min-p.
"""
import numpy as np
import pytest

import oracle
import top_select_gumbel_amd as ts
from top_select_gumbel_amd import workloads as wl
from gpu_helpers import GAP_EXEMPT, banner, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _torch():
    return torch_cuda()


def d32(a, dt):
    return None if a is None else dev(np.asarray(a, dt))


def run(x, k, p, t, mp, seeds):
    torch = torch_cuda()
    kept, mask, st = ts.ts_topp_mask_minp(dev(x), d32(k, np.int32), d32(p, np.float32), d32(t, np.float32),
                                          d32(mp, np.float32))
    tok, st2 = ts.ts_sample_rows_minp(dev(x), d32(k, np.int32), d32(p, np.float32), d32(t, np.float32),
                                      d32(mp, np.float32), dev(np.asarray(seeds, np.uint64)))
    torch.cuda.synchronize()
    assert np.array_equal(host(st), host(st2))
    return host(kept), host(mask), host(tok), host(st)


def check(x, k, p, t, mp, seeds, kept, mask, tok, st, label, row_ids=None):
    ids = list(range(x.shape[0])) if row_ids is None else list(row_ids)
    loose = 0
    for r in range(x.shape[0]):
        kr = None if k is None else int(k[r])
        pr = None if p is None else oracle.to_f32(p[r])
        tr = None if t is None else oracle.to_f32(t[r])
        o = oracle.sample_minp_row(x[r], kr, pr, tr, oracle.to_f32(mp[r]), int(seeds[r]), ids[r])
        tp = o.topp
        assert st[r] == o.status, f"{label} row {r}: status {st[r]} vs {o.status}"
        if o.status != 0:
            assert kept[r] == 0 and not mask[r].any() and tok[r] == -1
            continue
        kg = int(kept[r])
        if kg != tp.kept:
            assert (tp.minp_ambiguous or tp.ambiguous) and abs(kg - tp.kept) <= 3, \
                f"{label} row {r}: kept {kg} vs {tp.kept}"
            loose += 1
        ids_gpu = np.nonzero(mask[r])[0].tolist()
        assert len(ids_gpu) == kg and sorted(tp.order[:kg]) == ids_gpu, f"{label} row {r}: not the canonical prefix"
        want, gap = o.token, o.gap
        if kg != tp.kept and (tr is None or tr != 0.0):
            want, gap = oracle.gumbel_argmax(tp.x, tp.m, 1.0 if tr is None else tr, tp.order[:kg],
                                             int(seeds[r]), ids[r])
        if gap >= GAP_EXEMPT:
            assert tok[r] == want, f"{label} row {r}: token {tok[r]} vs {want} (gap {gap:.3g})"
    return loose


def test_minp_random_rows_and_status():
    rng = np.random.default_rng(61)
    v = 6000
    rows = 24
    x = (rng.standard_normal((rows, v)) * 2.5).astype(np.float32)
    x[3, :] = np.float32(1.0)                  # all equal
    x[4, 10] = np.nan                          # rejected
    k = rng.integers(1, 2500, rows).astype(np.int32)
    k[5:8] = v                                 # top-k off (row-streaming path; 7: full-row path without min-p)
    p = rng.uniform(0.5, 1.0, rows).astype(np.float32)
    p[7] = 1.0
    p[8] = 1.0
    t = rng.uniform(0.4, 1.6, rows).astype(np.float32)
    t[9] = 0.0                                 # greedy
    mp = rng.uniform(0.0, 0.3, rows).astype(np.float32)
    mp[0] = 0.0
    mp[10] = 1.0                               # only the maximum (and its ties) stay
    mp[11] = np.float32(-0.5)                  # invalid
    mp[12] = np.nan                            # invalid
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    banner("min-p random rows V=6000 (paths, greedy, invalid min_p)")
    kept, mask, tok, st = run(x, k, p, t, mp, seeds)
    check(x, k, p, t, mp, seeds, kept, mask, tok, st, "random")
    assert st[11] == ts.TS_ROW_BAD_MINP and st[12] == ts.TS_ROW_BAD_MINP


def test_minp_zero_matches_plain_entry_points():
    b = wl.decode(rows=16)
    mp = np.zeros(16, np.float32)
    banner("min-p = 0 against ts_topp_mask / ts_sample_rows (decode 16 rows)")
    kept, mask, tok, st = run(b.logits, b.k, b.p, b.t, mp, b.seeds)
    kept0, mask0, _ = ts.ts_topp_mask(dev(b.logits), dev(b.k), dev(b.p), dev(b.t))
    tok0, _ = ts.ts_sample_rows(dev(b.logits), dev(b.k), dev(b.p), dev(b.t), dev(b.seeds))
    assert np.array_equal(kept, host(kept0)) and np.array_equal(mask, host(mask0))
    assert np.array_equal(tok, host(tok0))


def test_minp_decode_rows_sampled():
    b = wl.decode()
    mp = np.full(64, 0.05, np.float32)
    banner("min-p 0.05 decode 64x151936 (12 rows checked)")
    kept, mask, tok, st = run(b.logits, b.k, b.p, b.t, mp, b.seeds)
    sel = list(range(0, 64, 6))
    check(b.logits[sel], b.k[sel], b.p[sel], b.t[sel], mp[sel], b.seeds[sel], kept[sel], mask[sel], tok[sel],
          st[sel], "decode", row_ids=sel)
    b = wl.decode_topp_only(rows=8)
    mp = np.full(8, 0.002, np.float32)
    banner("min-p 0.002 decode rows with top-k off 8x151936 (row-streaming path)")
    kept, mask, tok, st = run(b.logits, b.k, b.p, b.t, mp, b.seeds)
    check(b.logits, b.k, b.p, b.t, mp, b.seeds, kept, mask, tok, st, "topk-off")
