"""GPU parity of ts_sample_rows_logp (selected-token logprob and whole-row log-sum-exp)
against the binary64 oracle, through the C ABI.

Tolerance, from the arithmetic: each exponential is an fp32 exp2 of an argument formed in
fp32 from (x - m_w) and log2(e)/T, so its relative error is at most 2^-23 + 3 * 2^-24 * |y|
(y the base-2 exponent; terms below 2^-126 flush to 0, under 2^-100 of a share that holds
the maximum's 1); S is a mass-weighted average of those errors, below 2.5e-6 for any row of
these sizes (and near 1e-7 in practice); each wave share's rescaling to the row maximum is
fp32-accurate (about 1.5e-7 relative) and the logarithm is accurate to 1e-7 absolute, and the
final fp32 roundings add 2^-24 relative. Hence |delta| <= 3e-6 + 1.2e-7 * |value| for lse and
logp.
"""
import math

import numpy as np
import pytest

import oracle
import top_select_gumbel_amd as ts
from top_select_gumbel_amd import workloads as wl
from gpu_helpers import banner, dev, host, torch_cuda

pytestmark = pytest.mark.gpu
ATOL, RTOL = 3e-6, 1.2e-7


@pytest.fixture(scope="module", autouse=True)
def _torch():
    return torch_cuda()


def run(x, k, p, t, seeds):
    torch = torch_cuda()
    tok, logp, lse, st = ts.ts_sample_rows_logp(
        dev(x), None if k is None else dev(np.asarray(k, np.int32)),
        None if p is None else dev(np.asarray(p, np.float32)),
        None if t is None else dev(np.asarray(t, np.float32)), dev(np.asarray(seeds, np.uint64)))
    tok2, st2 = ts.ts_sample_rows(
        dev(x), None if k is None else dev(np.asarray(k, np.int32)),
        None if p is None else dev(np.asarray(p, np.float32)),
        None if t is None else dev(np.asarray(t, np.float32)), dev(np.asarray(seeds, np.uint64)))
    torch.cuda.synchronize()
    tok, tok2 = host(tok), host(tok2)
    assert np.array_equal(tok, tok2), "the logprob entry point samples the same tokens"
    assert np.array_equal(host(st), host(st2))
    return tok, host(logp), host(lse), host(st)


def check(x, t, tok, logp, lse, st, label, rows=None):
    rows = range(x.shape[0]) if rows is None else rows
    for r in rows:
        tv = 1.0 if t is None else oracle.to_f32(t[r])
        if st[r] != 0:
            assert math.isnan(logp[r]) and math.isnan(lse[r]), f"{label} row {r}: poisoned outputs"
            continue
        if tv == 0.0:
            assert logp[r] == 0.0 and lse[r] == np.inf, f"{label} row {r}: greedy"
            continue
        want_lse, want_lp = oracle.lse_logp_row(x[r], tv, int(tok[r]))
        assert abs(lse[r] - want_lse) <= ATOL + RTOL * abs(want_lse), \
            f"{label} row {r}: lse {lse[r]!r} vs {want_lse!r}"
        assert abs(logp[r] - want_lp) <= ATOL + RTOL * abs(want_lp), \
            f"{label} row {r}: logp {logp[r]!r} vs {want_lp!r}"
        assert logp[r] <= 0.0


def test_logp_tiny_and_v16():
    b = wl.tiny()
    banner("logp tiny")
    tok, lp, ls, st = run(b.logits, b.k, b.p, b.t, b.seeds)
    check(b.logits, b.t, tok, lp, ls, st, "tiny")
    b = wl.tiny_v16()
    banner("logp v16 x200 (ties, greedy rows, p = 1 rows)")
    tok, lp, ls, st = run(b.logits, b.k, b.p, b.t, b.seeds)
    check(b.logits, b.t, tok, lp, ls, st, "v16")


def test_logp_special_rows():
    rng = np.random.default_rng(44)
    v = 5000
    x = (rng.standard_normal((6, v)) * 3).astype(np.float32)
    x[1, ::2] = -np.inf                      # masked half
    x[2, 7] = np.nan                         # rejected
    x[3, :] = np.float32(2.5)                # all equal
    x[4, 100:] = -np.inf                     # 100 live tokens
    k = np.array([50, v, 10, 3000, v, v], np.int32)
    p = np.array([0.9, 0.95, 0.9, 0.5, 1.0, 0.7], np.float32)
    t = np.array([1.0, 0.8, 1.0, 1.3, 0.0, 2.0], np.float32)
    seeds = rng.integers(0, 2 ** 64, 6, dtype=np.uint64)
    banner("logp special rows (masked, NaN, all-equal, greedy)")
    tok, lp, ls, st = run(x, k, p, t, seeds)
    check(x, t, tok, lp, ls, st, "special")
    assert st[2] != 0


def test_logp_decode_and_paths():
    b = wl.decode()
    banner("logp decode 64x151936 (16 rows checked)")
    tok, lp, ls, st = run(b.logits, b.k, b.p, b.t, b.seeds)
    check(b.logits, b.t, tok, lp, ls, st, "decode", rows=range(0, 64, 4))
    b = wl.heavy(rows=8)
    banner("logp heavy-tailed 8x32000 (full-row path)")
    tok, lp, ls, st = run(b.logits, b.k, b.p, b.t, wl.heavy_launch_seeds(0, 8))
    check(b.logits, b.t, tok, lp, ls, st, "heavy")
    b = wl.decode_topp_only(rows=8)
    banner("logp decode rows with top-k off 8x151936 (row-streaming path)")
    tok, lp, ls, st = run(b.logits, b.k, b.p, b.t, b.seeds)
    check(b.logits, b.t, tok, lp, ls, st, "topk-off")


def test_logp_deterministic_and_batch_invariant():
    b = wl.decode(rows=16)
    banner("logp repeat + single-row batches")
    tok, lp, ls, st = run(b.logits, b.k, b.p, b.t, b.seeds)
    for _ in range(3):
        tok2, lp2, ls2, _ = run(b.logits, b.k, b.p, b.t, b.seeds)
        assert np.array_equal(tok, tok2) and np.array_equal(lp.view(np.uint32), lp2.view(np.uint32))
        assert np.array_equal(ls.view(np.uint32), ls2.view(np.uint32))
    for r in (0, 5, 15):
        # the sampled token depends on the row's index (Philox counter), lse does not
        _, _, ls1, _ = run(b.logits[r:r + 1], b.k[r:r + 1], b.p[r:r + 1], b.t[r:r + 1], b.seeds[r:r + 1])
        assert ls1.view(np.uint32)[0] == ls.view(np.uint32)[r]
