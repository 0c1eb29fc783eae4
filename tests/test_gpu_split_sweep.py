"""Seeded small sampling calls without a top-k array (top-k off on every row). The host sends
the top-p / min-p rows of a call of at most 6.4 M logits over rows of at most 100,000 to the
row kernel's split nucleus. Every output byte must equal the forced nucleus passes, a call
with a top-k array of k = V and the forced row-streaming path, for ts_sample_rows,
ts_sample_rows_minp and ts_sample_rows_logp; the sampled tokens, the statuses and the top-p
counts must match the oracle on every row. Cases vary the batch (1-40 rows: 8 down to 6 parts
per row), the vocabulary (12,289-100,000, ragged quads) and the rows: spread logits at four
scales, exact ties, masked tokens, dominant heads, a narrow near-uniform row, an all-equal row,
greedy rows, min-p-only rows, and NaN or +inf rows (status codes); every fourth case calls the
min-p entry point with no top-p array.
"""
import numpy as np
import pytest

import oracle_pool as op
import top_select_gumbel_amd as ts
from gpu_helpers import banner, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


def make_case(i):
    rng = np.random.default_rng(9300 + i)
    v = int(rng.integers(12289, 100001))
    rows = int(rng.integers(1, 41))
    x = np.empty((rows, v), np.float32)
    for r in range(rows):
        scale = float(rng.choice([0.05, 1.0, 2.5, 40.0]))
        row = scale * rng.standard_normal(v)
        style = int(rng.integers(0, 7))
        if style == 1:
            row = np.round(row, 1)                                         # exact ties
        elif style == 2:
            row[rng.choice(v, v // 10, replace=False)] = -np.inf           # masked tokens
        elif style == 3:
            row[rng.choice(v, 20, replace=False)] += 8.0 * max(scale, 1.0)   # dominant heads
        elif style == 4:
            row = 1.0 + 1e-6 * rng.standard_normal(v)                      # narrow
        elif style == 5:
            row[:] = 3.0                                                   # all equal
        x[r] = row
    if rows > 2 and i % 3 == 0:
        x[rows - 1, int(rng.integers(0, v))] = np.nan                      # status: non-finite
        x[rows - 2, int(rng.integers(0, v))] = np.inf
    p = np.where(rng.random(rows) < 0.25, 1.0, rng.uniform(0.05, 1.0, rows)).astype(np.float32)
    t = np.where(rng.random(rows) < 0.1, 0.0, rng.uniform(0.3, 2.0, rows)).astype(np.float32)
    mp = np.where(rng.random(rows) < 0.5, 0.0, rng.uniform(0.0, 0.3, rows)).astype(np.float32)
    mp[p == 1.0] = np.maximum(mp[p == 1.0], 0.01)                          # min-p-only rows
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    return x, p, t, mp, seeds


def four_ways(fn):
    """fn(k) on the default routing, the forced nucleus passes, a k = V array, and the forced
    row-streaming path (k = V array)."""
    torch = torch_cuda()
    out = []
    for use_k, exact, passes in ((False, 0, 0), (False, 0, 1), (True, 0, 0), (True, 1, 0)):
        old = ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, exact)
        oldp = ts.ts_debug_set(ts.TS_KNOB_NUCLEUS_PASSES, passes)
        try:
            res = fn(use_k)
            torch.cuda.synchronize()
            out.append([host(a) for a in res])
        finally:
            ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, old)
            ts.ts_debug_set(ts.TS_KNOB_NUCLEUS_PASSES, oldp)
    for j in (1, 2, 3):
        for a, b in zip(out[0], out[j]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"way {j} differs from the default routing"
    return out[0]


@pytest.mark.parametrize("i", range(12))
def test_split_sweep_without_top_k_array(i):
    x, p, t, mp, seeds = make_case(i)
    rows, v = x.shape
    label = f"split sweep {i} ({rows} x {v})"
    xs, pd, td, md, sd = dev(x), dev(p), dev(t), dev(mp), dev(seeds)
    kv = dev(np.full(rows, v, np.int32))
    banner(f"{label}: sample, min-p, logp")
    tok, st = four_ways(lambda use_k: ts.ts_sample_rows(xs, kv if use_k else None, pd, td, sd))
    pm = None if i % 4 == 1 else pd                                        # min-p alone: no top-p array
    four_ways(lambda use_k: ts.ts_sample_rows_minp(xs, kv if use_k else None, pm, td, md, sd))
    lt, _, _, _ = four_ways(lambda use_k: ts.ts_sample_rows_logp(xs, kv if use_k else None, pd, td, sd))
    assert np.array_equal(lt, tok), "the logprob entry point samples the same tokens"
    banner(f"{label}: oracle")
    kept, mask, st2 = ts.ts_topp_mask(xs, None, pd, td, True)
    torch_cuda().cuda.synchronize()
    kept = host(kept)
    op.check_topp(x, None, p, t, kept, host(mask), host(st2), label)
    op.check_samples(x, None, p, t, seeds, tok, st, kept, label)
