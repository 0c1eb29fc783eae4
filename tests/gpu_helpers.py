"""Shared helpers for the GPU parity tests: device transfer and the matching rules.

Matching rules for batched top-k, top-p and sampling:
  * top-k: out_idx bytes equal the oracle's for every row;
  * top-p: kept counts equal the oracle's (rows whose binary64 boundary the oracle cannot
    certify are exempt from equality but not from the mass bound); the kept set is a canonical
    prefix holding the row maximum; its binary64 mass is at least p*Z*(1 - 1e-6);
  * sampling: ids equal the oracle's unless the oracle's best two perturbed scores are within
    1e-4; when the kept sets differ the oracle's argmax over the GPU's kept set is used.
"""
import math

import numpy as np
import pytest

import oracle

GAP_EXEMPT = 1e-4
MASS_REL = 1e-6


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev(a, dtype=None):
    torch = torch_cuda()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint64:
        a = a.view(np.int64)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda:0")


def host(t):
    return t.detach().cpu().numpy()


def banner(msg):
    print(f"[case] {msg}", flush=True)


def check_topk(x, k, k_max, out, status, label=""):
    st_o, idx_o = oracle.topk_select(x, k, k_max)
    assert np.array_equal(status, st_o), f"{label}: status {status} vs {st_o}"
    bad = [r for r in range(x.shape[0]) if not np.array_equal(out[r], idx_o[r])]
    assert not bad, f"{label}: rows {bad[:5]} differ, e.g. gpu {out[bad[0]][:12]} oracle {idx_o[bad[0]][:12]}"


def check_topp(x, k, p, t, kept, mask, status, label="", max_count_mismatch=0):
    """Returns the per-row oracle results (ToppResult list)."""
    res = oracle.topp_mask(x, k, p, t)
    mism = []
    for r, o in enumerate(res):
        assert status[r] == o.status, f"{label} row {r}: status {status[r]} vs {o.status}"
        if o.status != 0:
            assert kept[r] == 0, f"{label} row {r}: poisoned kept {kept[r]}"
            if mask is not None:
                assert not mask[r].any(), f"{label} row {r}: poisoned mask not empty"
            continue
        kg = int(kept[r])
        if kg != o.kept:
            mism.append((r, kg, o.kept, o.ambiguous))
            assert o.ambiguous or abs(kg - o.kept) <= 3, f"{label} row {r}: kept {kg} vs {o.kept}"
        assert kg >= 1
        if mask is not None:
            ids = np.nonzero(mask[r])[0].tolist()
            assert len(ids) == kg, f"{label} row {r}: mask has {len(ids)} ids, kept {kg}"
            assert sorted(o.order[:kg]) == ids, f"{label} row {r}: kept set is not the canonical prefix"
        pv = 1.0 if p is None else oracle.to_f32(p[r])
        tv = 1.0 if t is None else oracle.to_f32(t[r])
        if tv != 0.0 and pv != 1.0 and o.weights:
            mass = math.fsum(o.weights[: min(kg, len(o.weights))])
            assert mass >= pv * o.z * (1 - MASS_REL), f"{label} row {r}: kept mass below p*Z"
    strict = [m for m in mism if not m[3]]
    assert len(strict) <= max_count_mismatch, f"{label}: kept-count mismatches {strict[:5]}"
    return res


def check_samples(x, k, p, t, seeds, tokens, status, kept_gpu=None, label="", row_ids=None):
    """row_ids: the rows' indices within the GPU call (the Philox counter word); default 0..n-1."""
    ids = list(range(x.shape[0])) if row_ids is None else [int(v) for v in row_ids]
    x = np.asarray(x, np.float32)
    res = [oracle.sample_row(x[r], None if k is None else int(k[r]),
                             None if p is None else oracle.to_f32(p[r]),
                             None if t is None else oracle.to_f32(t[r]), int(seeds[r]), ids[r])
           for r in range(x.shape[0])]
    exempt = 0
    for r, o in enumerate(res):
        assert status[r] == o.status, f"{label} row {r}: status {status[r]} vs {o.status}"
        if o.status != 0:
            assert tokens[r] == -1
            continue
        want, gap = o.token, o.gap
        if kept_gpu is not None and o.topp.kept != int(kept_gpu[r]) and (t is None or t[r] != 0):
            tv = 1.0 if t is None else oracle.to_f32(t[r])
            kept_ids = o.topp.order[: int(kept_gpu[r])]
            want, gap = oracle.gumbel_argmax(o.topp.x, o.topp.m, tv, kept_ids, int(seeds[r]), ids[r])
        if gap < GAP_EXEMPT:
            exempt += 1
            continue
        assert tokens[r] == want, f"{label} row {r}: token {tokens[r]} vs oracle {want} (gap {gap:.3g})"
    return res, exempt
