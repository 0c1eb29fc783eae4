"""Rows of at most 12288 logits run in the row kernel alone (the row loaded into LDS; no
stream kernel). The same inputs through the two-kernel path (TS_KNOB_DIRECT = 0) must give
the same top-k ids, kept counts, masks and tokens, and both must match the oracle (top-k
bit-exact, top-p counts, sampled ids outside near-ties). Covers the 4 x 1024 and 200 x 16
rows of the small configuration, ragged lengths, 8192- and 12288-logit rows and greedy / full-row /
rejected rows.
"""
import numpy as np
import pytest

import oracle
import top_select_gumbel_amd as ts
from top_select_gumbel_amd import workloads as wl
from gpu_helpers import banner, check_samples, check_topk, check_topp, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _torch():
    return torch_cuda()


def d(a, dt):
    return None if a is None else dev(np.asarray(a, dt))


def both(fn):
    """fn() under the direct path and under the two-kernel path."""
    torch = torch_cuda()
    out = []
    for direct in (1, 0):
        old = ts.ts_debug_set(ts.TS_KNOB_DIRECT, direct)
        try:
            res = fn()
            torch.cuda.synchronize()
            out.append([None if v is None else host(v) for v in res])
        finally:
            ts.ts_debug_set(ts.TS_KNOB_DIRECT, old)
    return out


def batches():
    yield wl.tiny()
    yield wl.tiny_v16()
    b = wl.small_random(51, 24, 8192, 2048, scale=2.0)
    b.t[::6] = 0.0                                   # greedy rows
    b.k[1::6] = 8192                                 # top-k off
    b.p[2::6] = 1.0
    b.k[2::6] = 8192                                 # full row
    b.logits[3, 77] = np.nan                         # rejected row
    yield b
    yield wl.small_random(52, 16, 3000, 1500, tie_levels=5)
    yield wl.small_random(53, 12, 12288, 2048, scale=1.5)


@pytest.mark.parametrize("idx", range(5))
def test_direct_matches_two_kernel_path_and_oracle(idx):
    b = list(batches())[idx]
    x = b.logits
    banner(f"direct vs two-kernel {b.name} {x.shape}")
    k_max = int(max(b.k.max(), 1)) if b.k is not None else 1
    k_max = min(k_max, x.shape[1])
    kk = np.minimum(b.k, k_max).astype(np.int32)
    (o1, s1), (o2, s2) = both(lambda: ts.ts_topk_select(dev(x), d(kk, np.int32), k_max))
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    check_topk(x, kk, k_max, o1, s1, f"{b.name} direct")
    (k1, m1, t1), (k2, m2, t2) = both(lambda: ts.ts_topp_mask(dev(x), d(b.k, np.int32), d(b.p, np.float32),
                                                             d(b.t, np.float32)))
    assert np.array_equal(k1, k2) and np.array_equal(m1, m2) and np.array_equal(t1, t2)
    check_topp(x, b.k, b.p, b.t, k1, m1, t1, f"{b.name} direct")
    seeds = dev(np.asarray(b.seeds, np.uint64))
    (a1, u1), (a2, u2) = both(lambda: ts.ts_sample_rows(dev(x), d(b.k, np.int32), d(b.p, np.float32),
                                                        d(b.t, np.float32), seeds))
    assert np.array_equal(u1, u2)
    full = (b.k >= x.shape[1]) & (b.p == 1.0) & (b.t != 0)
    assert np.array_equal(a1[~full], a2[~full])
    check_samples(x, b.k, b.p, b.t, b.seeds, a1, u1, label=f"{b.name} direct")


def test_direct_topk_rows_lengths_and_value_order():
    rng = np.random.default_rng(61)
    x = np.round(rng.standard_normal((40, 5000)), 2).astype(np.float32)
    lengths = rng.integers(0, 5200, 40).astype(np.int32)
    k = rng.integers(1, 600, 40).astype(np.int32)
    offs = rng.integers(0, 1000, 40).astype(np.int32)
    banner("direct top-k rows: lengths, offsets, value order")
    for order in (ts.TS_ORDER_INDEX, ts.TS_ORDER_VALUE):
        (o1, s1), (o2, s2) = both(lambda: ts.ts_topk_select_rows(dev(x), d(k, np.int32), 600, d(lengths, np.int32),
                                                                 order, d(offs, np.int32)))
        assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
        st, want = oracle.topk_select_rows(x, lengths, k, 600, order, offs)
        assert np.array_equal(s1, st) and np.array_equal(o1, want)
