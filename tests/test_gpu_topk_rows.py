"""GPU parity of ts_topk_select_rows (sparse-indexer rows: per-row lengths, index or value
order, id offsets) against the oracle, bit-exact, through the C ABI."""
import numpy as np
import pytest

import oracle
import oracle_pool as op
import top_select_gumbel_amd as ts
from top_select_gumbel_amd import workloads as wl
from gpu_helpers import banner, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _torch():
    return torch_cuda()


def run(x, k, k_max, lengths, order, offsets):
    torch = torch_cuda()
    out, st = ts.ts_topk_select_rows(dev(x), dev(np.asarray(k, np.int32)), k_max,
                                     None if lengths is None else dev(np.asarray(lengths, np.int32)), order,
                                     None if offsets is None else dev(np.asarray(offsets, np.int32)))
    torch.cuda.synchronize()
    return host(out), host(st)


def check(x, k, k_max, lengths, order, offsets, label, rows=None):
    out, st = run(x, k, k_max, lengths, order, offsets)
    sel = list(range(x.shape[0])) if rows is None else list(rows)
    st_o, out_o = oracle.topk_select_rows(x[sel], None if lengths is None else np.asarray(lengths)[sel],
                                          np.asarray(k)[sel], k_max, order,
                                          None if offsets is None else np.asarray(offsets)[sel])
    assert np.array_equal(st[sel], st_o), f"{label}: status {st[sel]} vs {st_o}"
    bad = [i for i, r in enumerate(sel) if not np.array_equal(out[r], out_o[i])]
    assert not bad, f"{label}: rows {[sel[i] for i in bad[:5]]} differ: gpu {out[sel[bad[0]]][:10]} oracle {out_o[bad[0]][:10]}"


def test_ragged_random_rows_both_orders():
    rng = np.random.default_rng(71)
    v = 20000
    rows = 16
    x = np.round(rng.standard_normal((rows, v)), 2).astype(np.float32)   # tie-heavy
    lengths = rng.integers(-5, v + 50, rows).astype(np.int32)
    lengths[0] = 0          # empty row
    lengths[1] = 3          # shorter than k
    lengths[2] = v          # whole row
    lengths[3] = 9000
    x[3, 9000:] = np.nan    # NaN past the length does not reject
    x[4, 5] = np.nan        # inside the length: rejected
    lengths[4] = 100
    k = rng.integers(1, 2100, rows).astype(np.int32)
    offsets = rng.integers(0, 1 << 24, rows).astype(np.int32)
    for order in (ts.TS_ORDER_INDEX, ts.TS_ORDER_VALUE):
        banner(f"topk rows ragged V=20000 order {order}")
        check(x, k, 2100, lengths, order, offsets, f"ragged order {order}")


def test_value_order_large_k_exact_path():
    rng = np.random.default_rng(72)
    x = rng.standard_normal((4, 30000)).astype(np.float32)
    k = np.array([6000, 2500, 5000, 4000], np.int32)
    lengths = np.array([30000, 20000, 4500, 29999], np.int32)
    banner("topk rows value order, k up to 6000 (row-streaming path)")
    check(x, k, 6000, lengths, ts.TS_ORDER_VALUE, None, "large-k value order")


def test_indexer_rows_ragged_transform():
    b = wl.indexer_rows()
    rng = np.random.default_rng(73)
    lengths = rng.integers(1000, 131072 + 1, 32).astype(np.int32)
    offsets = (np.arange(32) * 131072 % (1 << 30)).astype(np.int32)   # each row's start in a flat space
    banner("topk rows indexer 32x131072 k=2048, value order, ragged offsets (every row)")
    out, st = run(b.logits, b.k, 2048, lengths, ts.TS_ORDER_VALUE, offsets)
    args = [("indexer", r, b.logits[r], int(lengths[r]), int(b.k[r]), 2048, ts.TS_ORDER_VALUE, int(offsets[r]),
             out[r], int(st[r])) for r in range(32)]
    errs = [e for e in op.pool().map(op.topk_rows_row, args, chunksize=1) if e]
    assert not errs, "; ".join(errs[:4])


def test_null_lengths_match_plain_topk():
    rng = np.random.default_rng(74)
    x = rng.standard_normal((6, 50000)).astype(np.float32)
    k = rng.integers(1, 2049, 6).astype(np.int32)
    banner("topk rows without lengths = ts_topk_select")
    out, st = run(x, k, 2048, None, ts.TS_ORDER_INDEX, None)
    out0, st0 = ts.ts_topk_select(dev(x), dev(k), 2048)
    assert np.array_equal(out, host(out0)) and np.array_equal(st, host(st0))
