"""Rows whose top-k array entry reaches the row length (top-k off, seen on the device only) with
top-p or min-p on take the row kernel's split nucleus: up to 8 workgroups per row each weigh a
part of the row and draw its window tokens' Gumbel scores, and the last one to finish cuts the
nucleus. The parts per row follow the batch size (8 for a few rows, 1 from 256 rows up), so the
row counts below cover 8, 3, 2 and 1 parts. Every output byte must equal the nucleus passes of
a call without a top-k array (forced), the single-workgroup row-streaming path (forced exact)
and a call without a top-k array on the default routing (small sampling calls take the split
nucleus there too), and every row must match the oracle. Rows mix spread logits, bf16-like ties, a narrow near-uniform
row, masked tokens, heavy ties, a dominant head, and min-p-only rows (p = 1).
"""
import numpy as np
import pytest

import oracle_pool as op
import top_select_gumbel_amd as ts
from gpu_helpers import banner, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


def d(a, dt):
    return None if a is None else dev(np.asarray(a, dt))


def rows_for(seed, rows, vocab):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, vocab)) * 2.5
    for r in range(rows):
        style = r % 6
        if style == 1:
            x[r] = np.round(rng.standard_normal(vocab) * 1e5 / 1024) * 1024      # bf16-like ties
        elif style == 2:
            x[r] = 1.0 + 1e-6 * rng.standard_normal(vocab)                       # narrow
        elif style == 3:
            x[r, rng.choice(vocab, vocab // 3, replace=False)] = -np.inf         # masked tokens
        elif style == 4:
            x[r] = np.round(rng.standard_normal(vocab), 1)                       # heavy ties
        elif style == 5:
            x[r, rng.choice(vocab, 20, replace=False)] += 8.0                    # dominant heads
    x = x.astype(np.float32)
    k = np.where(rng.random(rows) < 0.5, vocab, vocab + 7).astype(np.int32)     # top-k off by value
    p = rng.uniform(0.3, 0.99, rows).astype(np.float32)
    p[rng.random(rows) < 0.15] = 1.0
    t = rng.uniform(0.5, 1.5, rows).astype(np.float32)
    mp = np.where(rng.random(rows) < 0.5, 0.0, rng.uniform(0.0, 0.2, rows)).astype(np.float32)
    mp[p == 1.0] = np.maximum(mp[p == 1.0], 0.02)                             # p = 1 rows: min-p on
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    return x, k, p, t, mp, seeds


def three_ways(fn):
    """fn(k or None) with the top-k array (split nucleus), without it on the nucleus passes
    (forced), with the top-k array on the forced row-streaming path, and without it on the
    default routing (the split nucleus for small sampling calls, else the nucleus passes)."""
    torch = torch_cuda()
    out = []
    for use_k, exact, passes in ((True, 0, 0), (False, 0, 1), (True, 1, 0), (False, 0, 0)):
        old = ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, exact)
        oldp = ts.ts_debug_set(ts.TS_KNOB_NUCLEUS_PASSES, passes)
        try:
            res = fn(use_k)
            torch.cuda.synchronize()
            out.append([None if v is None else host(v) for v in res])
        finally:
            ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, old)
            ts.ts_debug_set(ts.TS_KNOB_NUCLEUS_PASSES, oldp)
    return out


def same(outs, what):
    for j in (1, 2, 3):
        for a, b in zip(outs[0], outs[j]):
            assert np.array_equal(a, b), f"{what}: split differs from path {j}"


@pytest.mark.parametrize("rows,vocab", [(3, 151936), (70, 50000), (100, 30000), (260, 20000)])
def test_split_nucleus_matches_other_paths_and_oracle(rows, vocab):
    x, k, p, t, mp, seeds = rows_for(9100 + rows, rows, vocab)
    xs, kd, pd, td, sd = dev(x), d(k, np.int32), d(p, np.float32), d(t, np.float32), dev(seeds)
    label = f"split nucleus {rows}x{vocab}"
    banner(f"{label}: topp")
    # min-p off: the p == 1 rows are plain full rows there, on every path
    outs = three_ways(lambda use_k: ts.ts_topp_mask(xs, kd if use_k else None, pd, td, True))
    same(outs, "topp mask")
    kept, mask, st = outs[0]
    op.check_topp(x, k, p, t, kept, mask, st, label)
    banner(f"{label}: sample")
    outs = three_ways(lambda use_k: ts.ts_sample_rows(xs, kd if use_k else None, pd, td, sd))
    same(outs, "sample")
    tok, st2 = outs[0]
    op.check_samples(x, k, p, t, seeds, tok, st2, kept, label)
    banner(f"{label}: min-p")
    mpd = d(mp, np.float32)
    outs = three_ways(lambda use_k: ts.ts_topp_mask_minp(xs, kd if use_k else None, pd, td, mpd))
    same(outs, "min-p mask")
    outs = three_ways(lambda use_k: ts.ts_sample_rows_minp(xs, kd if use_k else None, pd, td, mpd, sd))
    same(outs, "min-p sample")
    banner(f"{label}: logp")
    outs = three_ways(lambda use_k: ts.ts_sample_rows_logp(xs, kd if use_k else None, pd, td, sd))
    same(outs, "logp")
    assert np.array_equal(outs[0][0], tok)


def test_split_nucleus_counted_twice_in_a_row():
    """The per-row part counter is cleared by every call: the same workspace serves calls of
    different batch sizes back to back."""
    torch = torch_cuda()
    x, k, p, t, mp, seeds = rows_for(9200, 40, 40000)
    ref = None
    for rows in (40, 7, 40):
        banner(f"split nucleus back-to-back call with {rows} rows")
        tok, st = ts.ts_sample_rows(dev(x[:rows]), d(k[:rows], np.int32), d(p[:rows], np.float32),
                                    d(t[:rows], np.float32), dev(seeds[:rows]))
        torch.cuda.synchronize()
        tok = host(tok)
        if ref is None:
            ref = tok
        assert np.array_equal(tok[:7], ref[:7]) if rows == 7 else np.array_equal(tok, ref)
        assert (host(st) == 0).all()


def test_split_nucleus_decode_rows_as_benched():
    """The decode rows with a top-k array of k = V (64 x 151936: 4 parts per row), as the
    decode_topp_only bench times them: the same bytes as the nucleus passes and the
    row-streaming path, and every row against the oracle."""
    from top_select_gumbel_amd import workloads as wl
    b = wl.decode_topp_only()
    x, k, p, t, seeds = b.logits, b.k, b.p, b.t, b.seeds
    xs, kd, pd, td, sd = dev(x), d(k, np.int32), d(p, np.float32), d(t, np.float32), dev(seeds)
    label = "split nucleus decode 64x151936"
    banner(f"{label}: topp")
    outs = three_ways(lambda use_k: ts.ts_topp_mask(xs, kd if use_k else None, pd, td, True))
    same(outs, "topp mask")
    kept, mask, st = outs[0]
    op.check_topp(x, k, p, t, kept, mask, st, label)
    banner(f"{label}: sample")
    outs = three_ways(lambda use_k: ts.ts_sample_rows(xs, kd if use_k else None, pd, td, sd))
    same(outs, "sample")
    tok, st2 = outs[0]
    op.check_samples(x, k, p, t, seeds, tok, st2, kept, label)
