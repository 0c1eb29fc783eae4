"""GPU edge cases of the three entry points against the oracle: an empty batch, vocabularies
of one to five tokens, and rows that start at addresses that are not 16-byte aligned (an odd
row stride: the stream kernel's element-wise load path) with ragged chunk tails. Every case
prints a [case] line first."""
import numpy as np
import pytest

import top_select_gumbel_amd as ts
from gpu_helpers import banner, check_samples, check_topk, check_topp, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


def _strided(x, pad):
    """A device view of x whose rows are `pad` floats apart beyond their length."""
    rows, v = x.shape
    buf = np.full((rows, v + pad), np.float32(7.0), np.float32)   # padding would win if read
    buf[:, :v] = x
    return dev(buf)[:, :v]


def test_empty_batch():
    torch = torch_cuda()
    banner("empty batch: rows = 0")
    x = dev(np.zeros((0, 1000), np.float32))
    k = dev(np.zeros(0, np.int32))
    p = dev(np.zeros(0, np.float32))
    t = dev(np.zeros(0, np.float32))
    s = dev(np.zeros(0, np.uint64))
    idx, st = ts.ts_topk_select(x, k, 8)
    kept, mask, st2 = ts.ts_topp_mask(x, k, p, t, True)
    tok, st3 = ts.ts_sample_rows(x, k, p, t, s)
    torch.cuda.synchronize()
    assert idx.shape == (0, 8) and st.numel() == 0 and kept.numel() == 0 and tok.numel() == 0
    assert st2.numel() == 0 and st3.numel() == 0 and mask.shape == (0, 1000)


@pytest.mark.parametrize("v", [1, 2, 3, 5])
def test_tiny_vocabularies(v):
    torch = torch_cuda()
    rng = np.random.default_rng(40 + v)
    rows = 24
    x = rng.standard_normal((rows, v)).astype(np.float32)
    x[0] = 1.0                                   # all equal
    x[1, 0] = -np.inf                            # a masked token
    k = rng.integers(1, v + 3, rows).astype(np.int32)
    p = np.where(np.arange(rows) % 3 == 0, 1.0, rng.uniform(0.2, 1.0, rows)).astype(np.float32)
    t = np.where(np.arange(rows) % 5 == 0, 0.0, rng.uniform(0.5, 1.5, rows)).astype(np.float32)
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    banner(f"tiny vocabulary V={v}: topk")
    idx, st = ts.ts_topk_select(dev(x), dev(k), v + 2)
    torch.cuda.synchronize()
    check_topk(x, k, v + 2, host(idx), host(st), f"V={v}")
    banner(f"tiny vocabulary V={v}: topp")
    kept, mask, st2 = ts.ts_topp_mask(dev(x), dev(k), dev(p), dev(t), True)
    torch.cuda.synchronize()
    kept = host(kept)
    check_topp(x, k, p, t, kept, host(mask), host(st2), f"V={v}")
    banner(f"tiny vocabulary V={v}: sample")
    tok, st3 = ts.ts_sample_rows(dev(x), dev(k), dev(p), dev(t), dev(seeds))
    torch.cuda.synchronize()
    check_samples(x, k, p, t, seeds, host(tok), host(st3), kept, f"V={v}")


@pytest.mark.parametrize("v,pad", [(20003, 7), (40001, 1), (3001, 3)])
def test_unaligned_rows_and_ragged_tails(v, pad):
    torch = torch_cuda()
    rng = np.random.default_rng(v + pad)
    rows = 6
    x = (rng.standard_normal((rows, v)) * 2.0).astype(np.float32)
    x[2, -1] = 30.0                              # the maximum in the last element of a ragged tail
    x[3, v // 2] = np.float32(12.0)
    k = np.array([1, 50, 700, 2048, v + 1, 3], np.int32)
    p = np.array([0.9, 0.7, 1.0, 0.95, 0.8, 0.5], np.float32)
    t = np.array([1.0, 0.7, 1.3, 1.0, 1.1, 0.0], np.float32)
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    xs = _strided(x, pad)
    banner(f"unaligned rows V={v} stride={v + pad}: topk")
    idx, st = ts.ts_topk_select(xs, dev(np.minimum(k, v).astype(np.int32)), 2048)
    torch.cuda.synchronize()
    check_topk(x, np.minimum(k, v), 2048, host(idx), host(st), f"unaligned {v}")
    banner(f"unaligned rows V={v} stride={v + pad}: topp")
    kept, mask, st2 = ts.ts_topp_mask(xs, dev(k), dev(p), dev(t), True)
    torch.cuda.synchronize()
    kept = host(kept)
    check_topp(x, k, p, t, kept, host(mask), host(st2), f"unaligned {v}")
    banner(f"unaligned rows V={v} stride={v + pad}: sample")
    tok, st3 = ts.ts_sample_rows(xs, dev(k), dev(p), dev(t), dev(seeds))
    torch.cuda.synchronize()
    check_samples(x, k, p, t, seeds, host(tok), host(st3), kept, f"unaligned {v}")


def test_long_rows_flat_gather_all_entry_points():
    """Rows of 400,003 logits (49 chunks, 196 wave slices: more than one gather batch per wave)
    with candidate totals from a few hundred to several thousand, so that the row kernel's flat
    gather runs with each of its per-thread item counts, in all three entry points."""
    torch = torch_cuda()
    rng = np.random.default_rng(4003)
    rows, v = 6, 400003
    x = (rng.standard_normal((rows, v)) * 1.5).astype(np.float32)
    x[3] = np.round(x[3], 2)                     # ties at the top-k boundary
    k = np.array([1, 64, 700, 1500, 2048, 2048], np.int32)
    p = np.array([0.9, 0.8, 0.95, 1.0, 0.7, 0.99], np.float32)
    t = np.array([1.0, 0.8, 1.2, 1.0, 0.6, 1.4], np.float32)
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    banner(f"long rows V={v}: topk")
    idx, st = ts.ts_topk_select(dev(x), dev(k), 2048)
    torch.cuda.synchronize()
    check_topk(x, k, 2048, host(idx), host(st), "long rows")
    banner(f"long rows V={v}: topp")
    kept, mask, st2 = ts.ts_topp_mask(dev(x), dev(k), dev(p), dev(t), True)
    torch.cuda.synchronize()
    kept = host(kept)
    check_topp(x, k, p, t, kept, host(mask), host(st2), "long rows")
    banner(f"long rows V={v}: sample")
    tok, st3 = ts.ts_sample_rows(dev(x), dev(k), dev(p), dev(t), dev(seeds))
    torch.cuda.synchronize()
    check_samples(x, k, p, t, seeds, host(tok), host(st3), kept, "long rows")


def test_million_logit_rows_flat_gather_widest_round():
    """Rows of 2^20 logits with k = 2048 publish about 9,700 candidates: more than 16 per
    thread, so the flat gather takes its widest per-thread round (24 items) in the sampling and
    top-p instantiations too, not only in top-k select."""
    torch = torch_cuda()
    rng = np.random.default_rng(4004)
    rows, v = 2, 1 << 20
    x = rng.standard_normal((rows, v)).astype(np.float32)
    x[1] = np.round(x[1], 3)                     # ties at the top-k boundary
    k = np.array([2048, 2048], np.int32)
    p = np.array([0.9, 1.0], np.float32)
    t = np.array([1.0, 0.8], np.float32)
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    banner(f"million-logit rows V={v}: topk")
    idx, st = ts.ts_topk_select(dev(x), dev(k), 2048)
    torch.cuda.synchronize()
    check_topk(x, k, 2048, host(idx), host(st), "million rows")
    banner(f"million-logit rows V={v}: topp")
    kept, mask, st2 = ts.ts_topp_mask(dev(x), dev(k), dev(p), dev(t), True)
    torch.cuda.synchronize()
    kept = host(kept)
    check_topp(x, k, p, t, kept, host(mask), host(st2), "million rows")
    banner(f"million-logit rows V={v}: sample")
    tok, st3 = ts.ts_sample_rows(dev(x), dev(k), dev(p), dev(t), dev(seeds))
    torch.cuda.synchronize()
    check_samples(x, k, p, t, seeds, host(tok), host(st3), kept, "million rows")


def test_constant_stretches_uniform_slices():
    """Rows holding stretches of one repeated value (V = 151936: chunks of 8000 logits, wave
    shares of 2000). A wave whose every element is one key publishes a uniform slice (no
    stored entries); a wave holding more candidates than its slice flags it overflowed and the
    row takes the exact path. Both must give the oracle's results in all three entry points."""
    torch = torch_cuda()
    rng = np.random.default_rng(5150)
    rows, v = 6, 151936
    x = rng.standard_normal((rows, v)).astype(np.float32)
    x[0, 0:6000] = 9.0                           # three whole wave shares, the row's top
    x[1, 1000:9000] = 9.0                        # unaligned: partial waves overflow their slices
    x[2] = np.float32(0.5)                       # all equal
    x[3, 8000:16000] = 3.0                       # a whole chunk, the top-k boundary inside it
    x[3, rng.choice(v, 20, replace=False)] += 8.0
    x[4, 144000:] = 4.0                          # the last chunk, whole and ragged
    x[5, 50000:58000] = -np.inf                  # a masked chunk below the threshold
    k = np.array([2048, 1000, 700, 2048, 300, 1024], np.int32)
    p = np.array([0.9, 0.95, 0.8, 0.99, 0.7, 0.9], np.float32)
    t = np.array([1.0, 0.7, 1.2, 1.0, 0.0, 1.1], np.float32)
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    banner(f"constant stretches V={v}: topk")
    idx, st = ts.ts_topk_select(dev(x), dev(k), 2048)
    torch.cuda.synchronize()
    check_topk(x, k, 2048, host(idx), host(st), "stretches")
    banner(f"constant stretches V={v}: topp")
    kept, mask, st2 = ts.ts_topp_mask(dev(x), dev(k), dev(p), dev(t), True)
    torch.cuda.synchronize()
    kept = host(kept)
    check_topp(x, k, p, t, kept, host(mask), host(st2), "stretches")
    banner(f"constant stretches V={v}: sample")
    tok, st3 = ts.ts_sample_rows(dev(x), dev(k), dev(p), dev(t), dev(seeds))
    torch.cuda.synchronize()
    check_samples(x, k, p, t, seeds, host(tok), host(st3), kept, "stretches")
