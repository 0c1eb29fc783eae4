"""Row-parallel oracle checks for the GPU parity tests (CPU side only; no GPU code here).

The binary64 oracle costs about 0.1 s per 150k-logit row, so whole batches (64 decode rows,
128 tie-stress rows, 32 indexer rows) are checked row by row in a process pool. Each worker
runs the oracle for one row AND compares it with the GPU's outputs for that row, returning
only a short verdict, so no oracle result crosses a process boundary.

The pool uses spawned interpreters (fresh child processes that never touch the GPU) and at
most 16 workers, the CPU share of a one-GPU machine. The comparisons are the matching rules of
gpu_helpers: top-k bytes equal; top-p counts equal unless the oracle flags the row (then
within 3), canonical-prefix masks, kept mass >= p*Z*(1 - 1e-6); sampled ids equal unless the
oracle's best two perturbed scores are within 1e-4, with the oracle's argmax over the GPU's
kept set when the kept counts differ.
"""
from __future__ import annotations

import atexit
import math
import multiprocessing as mp
import os

import numpy as np

import oracle

GAP_EXEMPT = 1e-4
MASS_REL = 1e-6
MAX_WORKERS = 16

_POOL = None


def pool():
    global _POOL
    if _POOL is None:
        n = max(1, min(MAX_WORKERS, os.cpu_count() or 1))
        _POOL = mp.get_context("spawn").Pool(n)
        atexit.register(_POOL.terminate)
    return _POOL


def _opt(v, cast):
    return None if v is None else cast(v)


# ----------------------------------------------------------------------------- per-row workers
def topk_row(args):
    """(label, r, x, k, k_max, out_row, status) -> error message or None."""
    label, r, x, k, k_max, out_row, status = args
    st, idx = oracle.topk_select_row(x, int(k), k_max)
    if int(status) != st:
        return f"{label} row {r}: status {int(status)} vs oracle {st}"
    if not np.array_equal(np.asarray(out_row), np.asarray(idx, np.int32)):
        bad = int(np.nonzero(np.asarray(out_row) != np.asarray(idx, np.int32))[0][0])
        return f"{label} row {r}: out_idx differs first at slot {bad}: gpu {list(out_row[bad:bad + 6])} oracle {idx[bad:bad + 6]}"
    return None


def topp_row(args):
    """(label, r, x, k, p, t, kept, mask_ids or None, status) ->
    (error or None, (gpu kept, oracle kept, oracle ambiguous) when the counts differ)."""
    label, r, x, k, p, t, kept, mask_ids, status = args
    o = oracle.topp_row(x, _opt(k, int), _opt(p, oracle.to_f32), _opt(t, oracle.to_f32))
    if int(status) != o.status:
        return f"{label} row {r}: status {int(status)} vs oracle {o.status}", None
    if o.status != 0:
        if int(kept) != 0:
            return f"{label} row {r}: poisoned kept {int(kept)}", None
        if mask_ids is not None and len(mask_ids):
            return f"{label} row {r}: poisoned mask not empty", None
        return None, None
    kg = int(kept)
    mism = None
    if kg != o.kept:
        mism = (kg, o.kept, o.ambiguous)
        if not o.ambiguous and abs(kg - o.kept) > 3:
            return f"{label} row {r}: kept {kg} vs oracle {o.kept}", mism
    if kg < 1:
        return f"{label} row {r}: kept {kg} < 1", mism
    if mask_ids is not None:
        ids = [int(i) for i in mask_ids]
        if len(ids) != kg:
            return f"{label} row {r}: mask has {len(ids)} ids, kept {kg}", mism
        if sorted(o.order[:kg]) != ids:
            return f"{label} row {r}: kept set is not the canonical prefix", mism
    pv = 1.0 if p is None else oracle.to_f32(p)
    tv = 1.0 if t is None else oracle.to_f32(t)
    if tv != 0.0 and pv != 1.0 and o.weights:
        mass = math.fsum(o.weights[: min(kg, len(o.weights))])
        if mass < pv * o.z * (1 - MASS_REL):
            return f"{label} row {r}: kept mass below p*Z", mism
    return None, mism


def sample_row(args):
    """(label, r, row_id, x, k, p, t, seed, token, status, gpu kept or None) ->
    (error or None, exempt: bool)."""
    label, r, row_id, x, k, p, t, seed, token, status, kept_gpu = args
    o = oracle.sample_row(x, _opt(k, int), _opt(p, oracle.to_f32), _opt(t, oracle.to_f32), int(seed), int(row_id))
    if int(status) != o.status:
        return f"{label} row {r}: status {int(status)} vs oracle {o.status}", False
    if o.status != 0:
        return (None if int(token) == -1 else f"{label} row {r}: poisoned token {int(token)}"), False
    want, gap = o.token, o.gap
    tv = 1.0 if t is None else oracle.to_f32(t)
    if kept_gpu is not None and o.topp.kept != int(kept_gpu) and tv != 0.0:
        kept_ids = o.topp.order[: int(kept_gpu)]
        want, gap = oracle.gumbel_argmax(o.topp.x, o.topp.m, tv, kept_ids, int(seed), int(row_id))
    if gap < GAP_EXEMPT:
        return None, True
    if int(token) != want:
        return f"{label} row {r}: token {int(token)} vs oracle {want} (gap {gap:.3g})", False
    return None, False


def topk_rows_row(args):
    """Indexer variant: (label, r, x, length, k, k_max, order, offset, out_row, status)."""
    label, r, x, length, k, k_max, order, offset, out_row, status = args
    st, idx = oracle.topk_select_rows_row(x, length, int(k), k_max, order, offset)
    if int(status) != st:
        return f"{label} row {r}: status {int(status)} vs oracle {st}"
    if not np.array_equal(np.asarray(out_row), np.asarray(idx, np.int32)):
        return f"{label} row {r}: out_idx differs"
    return None


# ----------------------------------------------------------------------------- batch drivers
def _get(a, r):
    return None if a is None else a[r]


def check_topk(x, k, k_max, out, status, label="", rows=None):
    rows = range(x.shape[0]) if rows is None else rows
    args = [(label, r, np.ascontiguousarray(x[r]), int(k[r]), k_max, np.asarray(out[r]), int(status[r]))
            for r in rows]
    errs = [e for e in pool().map(topk_row, args, chunksize=1) if e]
    assert not errs, f"{len(errs)} rows differ: " + "; ".join(errs[:4])


def check_topp(x, k, p, t, kept, mask, status, label="", max_count_mismatch=0, rows=None):
    """Returns the list of (row, gpu kept, oracle kept, ambiguous) count mismatches."""
    rows = range(x.shape[0]) if rows is None else rows
    args = [(label, r, np.ascontiguousarray(x[r]), _get(k, r), _get(p, r), _get(t, r), int(kept[r]),
             None if mask is None else np.nonzero(mask[r])[0], int(status[r])) for r in rows]
    out = pool().map(topp_row, args, chunksize=1)
    errs = [e for e, _ in out if e]
    assert not errs, f"{len(errs)} rows fail: " + "; ".join(errs[:4])
    mism = [(r,) + m for r, (_, m) in zip(rows, out) if m is not None]
    strict = [m for m in mism if not m[3]]
    assert len(strict) <= max_count_mismatch, f"{label}: kept-count mismatches {strict[:5]}"
    return mism


def check_samples(x, k, p, t, seeds, tokens, status, kept_gpu=None, label="", rows=None, row_ids=None):
    """row_ids[r]: the Philox row word of row r (its index within the GPU call; default r).
    Returns the number of near-tie exemptions."""
    rows = range(x.shape[0]) if rows is None else rows
    args = [(label, r, r if row_ids is None else int(row_ids[r]), np.ascontiguousarray(x[r]), _get(k, r),
             _get(p, r), _get(t, r), int(seeds[r]), int(tokens[r]), int(status[r]),
             None if kept_gpu is None else int(kept_gpu[r])) for r in rows]
    out = pool().map(sample_row, args, chunksize=1)
    errs = [e for e, _ in out if e]
    assert not errs, f"{len(errs)} rows fail: " + "; ".join(errs[:4])
    return sum(1 for _, ex in out if ex)
