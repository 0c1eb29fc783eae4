"""A seeded sweep of shapes and row mixes through the three entry points, each against the
oracle on every row (oracle side in the process pool).

Each case draws its vocabulary from one of five bands, so that together they reach every
launch path: a few tokens, direct mode (the row kernel alone, V <= 12,288), the two-kernel path
with few chunks, decode-sized rows, and rows of more wave slices than one gather batch (the
flat gather). Rows mix logit scales, exact ties (values rounded to a coarse grid), masked
tokens (-inf), constant stretches, dominant head tokens, top-k on and off (k > V), top-p on
and off, greedy rows (T = 0) and padded row strides. Every case prints a [case] line first.
"""
import numpy as np
import pytest

import oracle_pool as op
import top_select_gumbel_amd as ts
from gpu_helpers import banner, dev, host, torch_cuda

pytestmark = pytest.mark.gpu

BANDS = [(2, 64), (1000, 12288), (12289, 60000), (150000, 160000), (330000, 420000)]
K_MAX = 2048


def make_case(i):
    rng = np.random.default_rng(7100 + i)
    lo, hi = BANDS[i % len(BANDS)]
    v = int(rng.integers(lo, hi + 1))
    rows = int(rng.integers(1, 6))
    x = np.empty((rows, v), np.float32)
    for r in range(rows):
        scale = float(rng.choice([0.05, 1.0, 4.0, 40.0]))
        row = scale * rng.standard_normal(v)
        style = int(rng.integers(0, 6))
        if style == 1:
            row = np.round(row, 1)                                  # exact ties
        elif style == 2 and v > 8:
            row[rng.choice(v, max(1, v // 10), replace=False)] = -np.inf   # masked tokens
        elif style == 3 and v > 4:
            a = int(rng.integers(0, v - 1))
            row[a:a + int(rng.integers(1, max(2, v // 3)))] = row.max() + 1.0   # a constant stretch on top
        elif style == 4:
            row[rng.choice(v, min(v, 20), replace=False)] += 8.0 * max(scale, 1.0)   # dominant heads
        x[r] = row.astype(np.float32)
    k = rng.integers(1, min(v, K_MAX) + 1, rows).astype(np.int32)
    k[rng.random(rows) < 0.25] = v + int(rng.integers(0, 3))        # top-k off
    p = np.where(rng.random(rows) < 0.3, 1.0, rng.uniform(0.05, 1.0, rows)).astype(np.float32)
    t = np.where(rng.random(rows) < 0.15, 0.0, rng.uniform(0.3, 2.0, rows)).astype(np.float32)
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    pad = int(rng.choice([0, 0, 4, 7]))
    return x, k, p, t, seeds, pad


def device_rows(x, pad):
    if not pad:
        return dev(x)
    rows, v = x.shape
    buf = np.full((rows, v + pad), np.float32(1e30), np.float32)   # padding would win if read
    buf[:, :v] = x
    return dev(buf)[:, :v]


@pytest.mark.parametrize("i", range(30))
def test_sweep_all_entry_points(i):
    torch = torch_cuda()
    x, k, p, t, seeds, pad = make_case(i)
    rows, v = x.shape
    label = f"sweep {i} ({rows} x {v}, stride pad {pad})"
    xs = device_rows(x, pad)
    kt = np.minimum(k, v).astype(np.int32)                         # top-k select needs k <= V
    banner(f"{label}: topk")
    idx, st = ts.ts_topk_select(xs, dev(kt), K_MAX)
    torch.cuda.synchronize()
    op.check_topk(x, kt, K_MAX, host(idx), host(st), label)
    banner(f"{label}: topp")
    kept, mask, st2 = ts.ts_topp_mask(xs, dev(k), dev(p), dev(t), True)
    torch.cuda.synchronize()
    kept = host(kept)
    op.check_topp(x, k, p, t, kept, host(mask), host(st2), label)
    banner(f"{label}: sample")
    tok, st3 = ts.ts_sample_rows(xs, dev(k), dev(p), dev(t), dev(seeds))
    torch.cuda.synchronize()
    op.check_samples(x, k, p, t, seeds, host(tok), host(st3), kept, label)
