"""GPU parity of the three C-ABI entry points against the binary64 oracle.

Sizes span several workgroup chunks and ragged tails; the full-size workloads (decode
64 x 151936, tie stress 128 x 128256, indexer 32 x 131072) are checked on every row, the
oracle side running row-parallel in a process pool (oracle_pool). Every case prints a
[case] line first so a failure can be located.
"""
import math

import numpy as np
import pytest

import oracle
import top_select_gumbel_amd as ts
from top_select_gumbel_amd import workloads as wl
import oracle_pool as op
from gpu_helpers import banner, check_samples, check_topk, check_topp, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _torch():
    return torch_cuda()


def run_topk(x, k, k_max, stride_pad=0):
    torch = torch_cuda()
    rows, v = x.shape
    if stride_pad:
        buf = np.zeros((rows, v + stride_pad), np.float32)
        buf[:, :v] = x
        xt = dev(buf)[:, :v]
    else:
        xt = dev(x)
    out, st = ts.ts_topk_select(xt, dev(np.asarray(k, np.int32)), k_max)
    torch.cuda.synchronize()
    return host(out), host(st)


def run_topp(x, k, p, t, want_mask=True):
    torch = torch_cuda()
    kept, mask, st = ts.ts_topp_mask(dev(x), None if k is None else dev(np.asarray(k, np.int32)),
                                     None if p is None else dev(np.asarray(p, np.float32)),
                                     None if t is None else dev(np.asarray(t, np.float32)), want_mask)
    torch.cuda.synchronize()
    return host(kept), (host(mask) if mask is not None else None), host(st)


def run_sample(x, k, p, t, seeds):
    torch = torch_cuda()
    tok, st = ts.ts_sample_rows(dev(x), None if k is None else dev(np.asarray(k, np.int32)),
                                None if p is None else dev(np.asarray(p, np.float32)),
                                None if t is None else dev(np.asarray(t, np.float32)),
                                dev(np.asarray(seeds, np.uint64)))
    torch.cuda.synchronize()
    return host(tok), host(st)


# ----------------------------------------------------------------------------- noise
def test_noise_words_and_gumbel_match_oracle():
    banner("gumbel noise: 4096 tokens, 3 seeds")
    torch = torch_cuda()
    toks = np.concatenate([np.arange(0, 2048), np.random.default_rng(0).integers(0, 1 << 30, 2048)]).astype(np.int32)
    for seed, row in [(0, 0), (0xDEADBEEFCAFEF00D, 17), (2 ** 64 - 1, 65535)]:
        w, u, g = ts.ts_gumbel_noise(seed, row, dev(toks))
        torch.cuda.synchronize()
        w = host(w).view(np.uint32)
        want = oracle.token_words(seed, row, toks)
        assert np.array_equal(w, want)
        u = host(u)
        assert np.array_equal(u.astype(np.float64), np.array([oracle.uniform_from_word(int(v)) for v in want]))
        g = host(g).astype(np.float64)
        g_ref = np.array([oracle.gumbel_from_word(int(v)) for v in want])
        assert np.all(np.abs(g - g_ref) <= g_tol(g_ref))


def g_tol(g_ref):
    """Noise error bound: 1e-6 plus two fp32 ulps of g (one ulp of g is 1.9e-6 at g = 16).
    Score errors this small cannot reorder two perturbed scores that differ by more than
    the 1e-4 near-tie exemption of the sampling rule, so sampled ids stay comparable."""
    return 1e-6 + 2 * np.spacing(np.abs(g_ref).astype(np.float32)).astype(np.float64)


def test_noise_transform_over_every_magnitude_of_u():
    banner("gumbel transform: words over every power of two")
    torch = torch_cuda()
    base = [1, 2, 3, 255, 256, 257]
    words = set(base)
    for e in range(0, 32):
        for dlt in (-3, -2, -1, 0, 1, 2, 3):
            v = (1 << e) + dlt
            if 0 <= v < (1 << 32):
                words.add(v)
    for top in range(1, 600):                      # u -> 1: the upper clamp region
        words.add((1 << 32) - top * 97)
    rng = np.random.default_rng(3)
    words |= set(int(v) for v in rng.integers(0, 1 << 32, 20000, dtype=np.uint64))
    words = np.array(sorted(words), dtype=np.uint64).astype(np.uint32)
    u, g = ts.ts_noise_transform(dev(words.view(np.int32)))
    torch.cuda.synchronize()
    u, g = host(u).astype(np.float64), host(g).astype(np.float64)
    assert np.array_equal(u, np.array([oracle.uniform_from_word(int(v)) for v in words]))
    g_ref = np.array([oracle.gumbel_from_word(int(v)) for v in words])
    over = np.abs(g - g_ref) - g_tol(g_ref)
    worst = int(np.argmax(over))
    assert over.max() <= 0, f"word {words[worst]} u {u[worst]!r}: g {g[worst]!r} vs {g_ref[worst]!r}"


def test_noise_clamp_endpoints():
    # The two ends of the clamp in closed form: word 0 maps to u = 0, clamped up to 2^-32,
    # so g = -log(-log1p(-2^-32)) = -log(2^-32 + 2^-65 + ...) = 32 ln 2 - ... ~ 22.18; the
    # largest word rounds to u = 1, clamped down to 1 - 2^-24, so g = -log(24 ln 2) ~ -2.81.
    # Words next to them stay inside the clamp.
    banner("gumbel noise: clamp end points in closed form")
    torch = torch_cuda()
    words = np.array([0, 1, 2, 0xFFFFFFFF, 0xFFFFFF80, 0xFFFFFF7F], dtype=np.uint64).astype(np.uint32)
    u, g = ts.ts_noise_transform(dev(words.view(np.int32)))
    torch.cuda.synchronize()
    u, g = host(u).astype(np.float64), host(g).astype(np.float64)
    lo, hi = 2.0 ** -32, 1.0 - 2.0 ** -24
    assert u[0] == lo and u[1] == lo and u[2] == 2.0 ** -31
    assert u[3] == hi and u[4] == hi and u[5] == hi
    g_lo = -math.log(-math.log1p(-lo))
    g_hi = -math.log(-math.log1p(-hi))
    assert abs(g_lo - 32 * math.log(2)) < 1e-8 and abs(g_hi + math.log(24 * math.log(2))) < 1e-6
    ref = np.array([g_lo, g_lo, -math.log(-math.log1p(-2.0 ** -31)), g_hi, g_hi, g_hi])
    assert np.all(np.abs(g - ref) <= g_tol(ref)), (g, ref)


# ----------------------------------------------------------------------------- top-k
def test_topk_tiny_config():
    b = wl.tiny()
    banner("topk tiny 4x1024 k=50")
    out, st = run_topk(b.logits, b.k, 50)
    check_topk(b.logits, b.k, 50, out, st, "tiny")


def test_topk_v16_rows():
    b = wl.tiny_v16()
    banner("topk 200 rows V=16")
    out, st = run_topk(b.logits, b.k, 16)
    check_topk(b.logits, b.k, 16, out, st, "v16")


@pytest.mark.parametrize("rows,v,k_hi,kind,pad", [
    (8, 50000, 2048, "normal", 0),
    (5, 100003, 700, "normal", 5),            # ragged vocab, unaligned rows
    (6, 81920, 2048, "ties", 0),              # heavy exact ties
    (3, 40961, 100, "normal", 3),             # one element past a chunk
    (7, 4097, 5000, "normal", 0),             # k >= V for some rows
])
def test_topk_random(rows, v, k_hi, kind, pad):
    banner(f"topk random rows={rows} V={v} k<= {k_hi} kind={kind} pad={pad}")
    b = wl.small_random(100 + rows, rows, v, k_hi, tie_levels=7 if kind == "ties" else 0)
    k_max = k_hi
    out, st = run_topk(b.logits, b.k, k_max, stride_pad=pad)
    check_topk(b.logits, b.k, k_max, out, st, kind)


def test_topk_special_rows():
    banner("topk special rows")
    v = 3000
    x = np.random.default_rng(1).standard_normal((9, v)).astype(np.float32)
    x[0] = 2.5                                  # all equal -> [0, k)
    x[1, ::2] = -0.0
    x[1, 1::2] = 0.0                            # signed zeros tie
    x[2] = np.float32(1e-40) * np.arange(v)     # subnormals are distinct keys
    x[3, 17] = np.nan                           # rejected
    x[4, 5] = np.inf                            # +-inf are ordinary keys
    x[4, 6] = -np.inf
    x[5] = -np.inf
    x[6] = np.float32(3e38) * np.sign(np.random.default_rng(2).standard_normal(v)).astype(np.float32)
    x[7, :] = np.float32(1.0) + np.float32(2.0 ** -23) * (np.arange(v) % 3)   # adjacent fp32 values
    k = np.array([77, 1500, 100, 5, 10, 20, 2000, 999, 0], np.int32)
    out, st = run_topk(x, k, 2048)
    check_topk(x, k, 2048, out, st, "special")


def test_topk_large_k_stream_path():
    banner("topk k up to 6000 (row-streaming path)")
    b = wl.small_random(7, 4, 30000, 6000)
    out, st = run_topk(b.logits, b.k, 6000)
    check_topk(b.logits, b.k, 6000, out, st, "large-k")


def test_topk_indexer_rows_every_row():
    b = wl.indexer_rows()
    banner("topk indexer 32x131072 k=2048 (every row)")
    out, st = run_topk(b.logits, b.k, 2048)
    op.check_topk(b.logits, b.k, 2048, out, st, "indexer")


def test_topk_indexer_long_and_near_uniform():
    for b in (wl.indexer_long(), wl.indexer_near_uniform()):
        banner(f"topk {b.name} {b.logits.shape}")
        out, st = run_topk(b.logits, b.k, 2048)
        check_topk(b.logits, b.k, 2048, out, st, b.name)


def test_topk_long_rows_global_candidates():
    # 1M-element rows, k=2048. Row 0 publishes about 9,700 candidates: they fit in LDS with
    # the automatic 8192-logit chunks; with 4096-logit chunks (twice the workgroups, so twice
    # the per-workgroup safety margins) about 14,000 do not, and the row takes the filtered
    # gather from the slices in global memory. Row 1 has 40000 ties at its maximum, so every
    # candidate key is equal and the first k by id are taken; row 2 puts 20000 items on each
    # of two adjacent fp32 values, the filtered set is still too large and the row takes the
    # exact path from the smallest workgroup threshold.
    rng = np.random.default_rng(91)
    n = 1 << 20
    x = np.round(rng.standard_normal((3, n)), 3).astype(np.float32)
    x[1, rng.choice(n, 40000, replace=False)] = np.float32(9.0)
    v0 = np.float32(7.0)
    v1 = np.nextafter(v0, np.float32(8.0))
    pos = rng.choice(n, 40000, replace=False)
    x[2, pos[:20000]] = v0
    x[2, pos[20000:]] = v1
    k = np.array([2048, 2048, 2048], np.int32)
    banner("topk 3x1048576 k=2048: filtered gather, all-equal cut, exact fallback")
    out, st = run_topk(x, k, 2048)
    check_topk(x, k, 2048, out, st, "long")
    try:
        ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 4096)
        out2, st2 = run_topk(x, k, 2048)
    finally:
        ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 0)
    assert np.array_equal(out2, out) and np.array_equal(st2, st)


def test_topk_deterministic_and_path_invariant():
    banner("topk repeat + chunk-size forcing")
    b = wl.small_random(9, 6, 90000, 2048, tie_levels=50)
    ref, _ = run_topk(b.logits, b.k, 2048)
    for _ in range(5):
        out, _ = run_topk(b.logits, b.k, 2048)
        assert np.array_equal(out, ref)
    try:
        # 64- and 256-element chunks give more wave slices than the row kernel indexes and
        # take the exact row-streaming path; the others the candidate path
        for ce in (64, 256, 1024, 2048, 4096, 8192):
            ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, ce)
            out, _ = run_topk(b.logits, b.k, 2048)
            assert np.array_equal(out, ref), f"chunk {ce}"
        ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 0)
        ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, 1)
        out, _ = run_topk(b.logits, b.k, 2048)
        assert np.array_equal(out, ref), "exact row-streaming path"
    finally:
        ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 0)
        ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, 0)


# ----------------------------------------------------------------------------- top-p
def test_topp_tiny_and_v16():
    b = wl.tiny()
    banner("topp tiny")
    kept, mask, st = run_topp(b.logits, b.k, b.p, b.t)
    check_topp(b.logits, b.k, b.p, b.t, kept, mask, st, "tiny")
    b = wl.tiny_v16()
    banner("topp v16 x200")
    kept, mask, st = run_topp(b.logits, b.k, b.p, b.t)
    check_topp(b.logits, b.k, b.p, b.t, kept, mask, st, "v16")


@pytest.mark.parametrize("rows,v,k_hi,scale,ties", [
    (16, 30000, 2048, 2.0, 0),
    (8, 70001, 1024, 3.0, 0),
    (8, 50000, 1500, 1.0, 5),
])
def test_topp_random(rows, v, k_hi, scale, ties):
    banner(f"topp random rows={rows} V={v} k<={k_hi}")
    b = wl.small_random(200 + rows, rows, v, k_hi, scale=scale, tie_levels=ties)
    kept, mask, st = run_topp(b.logits, b.k, b.p, b.t)
    check_topp(b.logits, b.k, b.p, b.t, kept, mask, st, "random")


def test_topp_topk_off_and_special():
    banner("topp with top-k off (stream path), T=0, p=1, invalid rows")
    rng = np.random.default_rng(5)
    v = 12000
    x = (rng.standard_normal((10, v)) * 1.5).astype(np.float32)
    x[3, 100] = np.inf
    x[4] = -np.inf
    x[5, :50] = -np.inf
    p = np.array([0.9, 0.5, 1.0, 0.9, 0.9, 0.95, 0.0, 0.7, 0.8, 0.99], np.float32)
    t = np.array([1.0, 0.7, 1.0, 1.0, 1.0, 1.3, 1.0, 0.0, -1.0, 1.0], np.float32)
    kept, mask, st = run_topp(x, None, p, t)
    check_topp(x, None, p, t, kept, mask, st, "k-off")
    k = np.array([3000, 1, 5, 12000, 100, 2500, 10, 10, 10, 4000], np.int32)
    kept, mask, st = run_topp(x, k, p, t)
    check_topp(x, k, p, t, kept, mask, st, "k-mixed")


def test_topp_decode_every_row():
    b = wl.decode()
    banner("topp decode 64x151936 (every row, masks)")
    kept, mask, st = run_topp(b.logits, b.k, b.p, b.t, want_mask=True)
    op.check_topp(b.logits, b.k, b.p, b.t, kept, mask, st, "decode")


def test_topp_and_sample_decode_topk_off_every_row():
    # top-p over whole 151936-element rows (top-k disabled): the nucleus passes, or with a
    # top-k array of k = V the per-row path
    b = wl.decode_topp_only()                 # a top-k array holding k = V
    banner("topp + sample decode with k off 64x151936 (every row)")
    kept, mask, st = run_topp(b.logits, b.k, b.p, b.t, want_mask=True)
    tok, st2 = run_sample(b.logits, b.k, b.p, b.t, b.seeds)
    op.check_topp(b.logits, b.k, b.p, b.t, kept, mask, st, "topk-off")
    op.check_samples(b.logits, b.k, b.p, b.t, b.seeds, tok, st2, kept, "topk-off")
    # no top-k array at all: the same bytes
    kept2, mask2, st3 = run_topp(b.logits, None, b.p, b.t, want_mask=True)
    tok2, _ = run_sample(b.logits, None, b.p, b.t, b.seeds)
    assert np.array_equal(kept2, kept) and np.array_equal(mask2, mask) and np.array_equal(st3, st)
    assert np.array_equal(tok2, tok)


def test_tie_stress_every_row():
    # bf16-rounded logits at 1e5 scale (exact ties everywhere) and one all-equal row (the
    # last): top-k bytes, top-p counts and masks, and sampled ids on all 128 rows
    b = wl.tie_stress()
    banner("tie stress 128x128256: topk + topp + sample (every row, incl. the all-equal row)")
    out, st0 = run_topk(b.logits, b.k, 2048)
    op.check_topk(b.logits, b.k, 2048, out, st0, "tie topk")
    assert out[127, : b.k[127]].tolist() == list(range(b.k[127]))      # all equal: ids [0, k)
    kept, mask, st = run_topp(b.logits, b.k, b.p, b.t, want_mask=True)
    op.check_topp(b.logits, b.k, b.p, b.t, kept, mask, st, "tie topp")
    tok, st2 = run_sample(b.logits, b.k, b.p, b.t, b.seeds)
    exempt = op.check_samples(b.logits, b.k, b.p, b.t, b.seeds, tok, st2, kept, "tie sample")
    assert exempt <= 4


# ----------------------------------------------------------------------------- sampling
def test_sample_tiny_and_v16():
    b = wl.tiny()
    banner("sample tiny")
    tok, st = run_sample(b.logits, b.k, b.p, b.t, b.seeds)
    kept, _, _ = run_topp(b.logits, b.k, b.p, b.t, want_mask=False)
    check_samples(b.logits, b.k, b.p, b.t, b.seeds, tok, st, kept, "tiny")
    b = wl.tiny_v16()
    banner("sample v16 x200")
    tok, st = run_sample(b.logits, b.k, b.p, b.t, b.seeds)
    kept, _, _ = run_topp(b.logits, b.k, b.p, b.t, want_mask=False)
    check_samples(b.logits, b.k, b.p, b.t, b.seeds, tok, st, kept, "v16")


def test_sample_random_and_paths():
    rng = np.random.default_rng(77)
    v = 20000
    x = (rng.standard_normal((12, v)) * 2).astype(np.float32)
    x[11, :] = -np.inf
    k = np.array([5, 2048, 100, 20000, 20000, 20000, 3000, 1, 700, 20000, 64, 10], np.int32)
    p = np.array([0.9, 0.8, 1.0, 1.0, 0.9, 1.0, 0.95, 0.5, 0.6, 1.0, 0.99, 0.9], np.float32)
    t = np.array([1.0, 0.6, 1.2, 1.0, 1.0, 0.0, 1.0, 1.0, 1.0, 1.4, 0.5, 1.0], np.float32)
    seeds = rng.integers(0, 2 ** 64, 12, dtype=np.uint64)
    banner("sample mixed paths V=20000")
    tok, st = run_sample(x, k, p, t, seeds)
    kept, _, _ = run_topp(x, k, p, t, want_mask=False)
    check_samples(x, k, p, t, seeds, tok, st, kept, "mixed")


def test_sample_decode_every_row():
    b = wl.decode()
    banner("sample decode 64x151936 (every row)")
    tok, st = run_sample(b.logits, b.k, b.p, b.t, b.seeds)
    kept, _, _ = run_topp(b.logits, b.k, b.p, b.t, want_mask=False)
    exempt = op.check_samples(b.logits, b.k, b.p, b.t, b.seeds, tok, st, kept, "decode")
    assert exempt <= 2


def test_sample_heavy_rows_match_oracle():
    b = wl.heavy(rows=8)
    seeds = wl.heavy_launch_seeds(0, 8)
    banner("sample heavy-tailed 8x32000 (full-row path)")
    tok, st = run_sample(b.logits, b.k, b.p, b.t, seeds)
    check_samples(b.logits, b.k, b.p, b.t, seeds, tok, st, None, "heavy")


def test_topp_and_sample_long_rows_global_candidates():
    # 1M-element rows: the candidates fit in LDS with the automatic chunks; with 4096-logit
    # chunks they exceed it, and top-p and sampling run after the filtered gather from global
    # memory. Both must give the same bytes.
    rng = np.random.default_rng(92)
    n = 1 << 20
    x = (rng.standard_normal((2, n)) * 2.5).astype(np.float32)
    k = np.array([2048, 1500], np.int32)
    p = np.array([0.9, 0.97], np.float32)
    t = np.array([1.0, 0.7], np.float32)
    seeds = rng.integers(0, 2 ** 64, 2, dtype=np.uint64)
    banner("topp + sample 2x1048576 k=2048/1500 (filtered gather)")
    kept, mask, st = run_topp(x, k, p, t, want_mask=True)
    check_topp(x, k, p, t, kept, mask, st, "long")
    tok, st = run_sample(x, k, p, t, seeds)
    check_samples(x, k, p, t, seeds, tok, st, kept, "long")
    try:
        ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 4096)
        kept2, mask2, _ = run_topp(x, k, p, t, want_mask=True)
        tok2, _ = run_sample(x, k, p, t, seeds)
    finally:
        ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 0)
    assert np.array_equal(kept2, kept) and np.array_equal(mask2, mask) and np.array_equal(tok2, tok)


def test_sample_deterministic_and_path_invariant():
    banner("sample repeat + chunk forcing")
    b = wl.small_random(31, 8, 100000, 2048, scale=2.0)
    ref, _ = run_sample(b.logits, b.k, b.p, b.t, b.seeds)
    kref, mref, _ = run_topp(b.logits, b.k, b.p, b.t)
    for _ in range(3):
        tok, _ = run_sample(b.logits, b.k, b.p, b.t, b.seeds)
        assert np.array_equal(tok, ref)
    try:
        for ce, exact in ((256, 0), (1024, 0), (3072, 0), (0, 1)):
            ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, ce)
            ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, exact)
            tok, _ = run_sample(b.logits, b.k, b.p, b.t, b.seeds)
            assert np.array_equal(tok, ref), f"chunk {ce} exact {exact}"
            kept, mask, _ = run_topp(b.logits, b.k, b.p, b.t)
            assert np.array_equal(kept, kref) and np.array_equal(mask, mref)
    finally:
        ts.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 0)
        ts.ts_debug_set(ts.TS_KNOB_FORCE_EXACT, 0)
