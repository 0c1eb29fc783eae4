"""Pins for the oracle's Philox4x32-10 stream and Gumbel noise map (CPU only).

* Philox: checked against an independent implementation of the same published
  generator (Triton's Philox, run by its CPU interpreter; skipped when Triton is not
  importable), and the scalar and vectorised oracle versions against each other.
* Noise: g = -log(-log1p(-u)) (vLLM PR #45996 summary, "key source excerpts") is pinned
  by the Gumbel CDF written the other way round: F(g) = exp(-exp(-g)) must equal 1 - u,
  i.e. the large-noise tail sits at u -> 0 where fp32 has resolution. The clamp end
  points are closed forms.
"""
import math
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle
from oracle import philox as ph


def test_vectorised_matches_scalar():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 2 ** 32, size=(4, 64), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    vec = ph.philox4x32_np(c[0], c[1], c[2], c[3], k0, k1)
    for j in range(64):
        want = ph.philox4x32((c[0, j], c[1, j], c[2, j], c[3, j]), (k0, k1))
        assert tuple(int(v[j]) for v in vec) == want


def test_zero_rounds_is_identity_and_rounds_mix():
    assert ph.philox4x32((1, 2, 3, 4), (5, 6), rounds=0) == (1, 2, 3, 4)
    a = ph.philox4x32((0, 0, 0, 0), (0, 0))
    b = ph.philox4x32((1, 0, 0, 0), (0, 0))
    diff = sum(bin(x ^ y).count("1") for x, y in zip(a, b))
    assert 40 < diff < 88                                   # avalanche: ~64 of 128 bits flip


def test_seed_key_split():
    assert ph.seed_key(0x0123456789ABCDEF) == (0x89ABCDEF, 0x01234567)


def test_token_word_layout():
    seed, row = 0xDEADBEEFCAFEF00D, 17
    toks = np.arange(0, 40)
    words = ph.token_words(seed, row, toks)
    k0, k1 = ph.seed_key(seed)
    for t in toks:
        blk = ph.philox4x32((t >> 2, row, 0, 0), (k0, k1))
        assert int(words[t]) == blk[t & 3]


TRITON_SCRIPT = textwrap.dedent("""
    import os, sys, json
    os.environ["TRITON_INTERPRET"] = "1"
    import torch, triton, triton.language as tl

    @triton.jit
    def _k(out, seed, c0p, c1p, N: tl.constexpr):
        o = tl.arange(0, N)
        c0 = tl.load(c0p + o)
        c1 = tl.load(c1p + o)
        z = c0 * 0
        a, b, c, d = tl.philox(seed, c0, c1, z, z, 10)
        tl.store(out + o * 4 + 0, a)
        tl.store(out + o * 4 + 1, b)
        tl.store(out + o * 4 + 2, c)
        tl.store(out + o * 4 + 3, d)

    cases = json.loads(sys.argv[1])
    res = []
    for seed, c0s, c1s in cases:
        n = len(c0s)
        out = torch.zeros(4 * n, dtype=torch.int32)
        c0 = torch.tensor([v - (1 << 32) if v >= (1 << 31) else v for v in c0s], dtype=torch.int32)
        c1 = torch.tensor([v - (1 << 32) if v >= (1 << 31) else v for v in c1s], dtype=torch.int32)
        _k[(1,)](out, seed, c0, c1, n)
        res.append([v & 0xFFFFFFFF for v in out.tolist()])
    print(json.dumps(res))
""")


def test_philox_matches_independent_triton_interpreter():
    pytest.importorskip("triton")
    import json
    rng = np.random.default_rng(21)
    cases = []
    for seed in [0, 1, 0xFFFFFFFFFFFFFFFF, 0x5EED0000, int(rng.integers(0, 2 ** 63))]:
        c0 = [0, 1, 2, 0xFFFFFFFF, int(rng.integers(0, 2 ** 32)), int(rng.integers(0, 2 ** 32)), 7, 8]
        c1 = [0, 0, 5, 0xFFFFFFFF, int(rng.integers(0, 2 ** 32)), 3, 255, 65535]
        cases.append([seed, c0, c1])
    env = dict(os.environ, TRITON_INTERPRET="1")
    try:
        out = subprocess.run([sys.executable, "-c", TRITON_SCRIPT, json.dumps(cases)],
                             capture_output=True, text=True, env=env, timeout=600)
    except subprocess.TimeoutExpired:
        pytest.skip("Triton interpreter timed out")
    if out.returncode != 0:
        pytest.skip("Triton interpreter unavailable: " + out.stderr[-300:])
    got = json.loads(out.stdout.strip().splitlines()[-1])
    for (seed, c0, c1), words in zip(cases, got):
        k0, k1 = ph.seed_key(seed)
        for j in range(len(c0)):
            assert tuple(words[4 * j: 4 * j + 4]) == ph.philox4x32((c0[j], c1[j], 0, 0), (k0, k1))


def test_words_are_uniform_chi_square():
    from scipy.stats import chisquare
    w = ph.token_words(12345, 3, np.arange(200000))
    counts = np.bincount((w >> 24).astype(np.int64), minlength=256)
    assert chisquare(counts).pvalue > 1e-4


def test_noise_inverts_the_gumbel_cdf():
    rng = np.random.default_rng(4)
    words = rng.integers(1, 2 ** 32 - 256, size=5000)
    for wd in words:
        u = oracle.uniform_from_word(int(wd))
        g = oracle.gumbel_from_word(int(wd))
        # 1 - F(g) computed with expm1/exp, not log1p/log
        tail = -math.expm1(-math.exp(-g))
        assert tail == pytest.approx(u, rel=1e-12)


def test_uniform_map_is_fp32_rounding_and_clamped():
    assert oracle.uniform_from_word(0) == 2.0 ** -32
    assert oracle.uniform_from_word(1) == 2.0 ** -32
    assert oracle.uniform_from_word(2 ** 32 - 1) == 1.0 - 2.0 ** -24      # 1 - 2^-32 rounds to 1
    assert oracle.uniform_from_word(2 ** 31) == 0.5
    # 2^24 + 1 is not an fp32 value: (2^24 + 1) * 2^-32 rounds to even, i.e. 2^24 * 2^-32
    assert oracle.uniform_from_word(2 ** 24 + 1) == 2.0 ** -8
    assert oracle.uniform_from_word(2 ** 24 + 3) == (2 ** 24 + 4) * 2.0 ** -32


def test_noise_clamp_endpoints_closed_form():
    # u = 2^-32: -log1p(-u) = u (1 + u/2 + ...), so g = 32 ln 2 - u/2 to first order
    assert oracle.gumbel_from_word(0) == pytest.approx(32 * math.log(2) - 2.0 ** -33, rel=1e-14)
    assert oracle.gumbel_from_word(2 ** 32 - 1) == pytest.approx(-math.log(24 * math.log(2)), rel=1e-12)


def test_noise_mean_is_euler_gamma():
    w = ph.token_words(999, 0, np.arange(100000))
    g = np.array([oracle.gumbel_from_word(int(v)) for v in w])
    assert abs(g.mean() - 0.5772156649) < 5 * (math.pi / math.sqrt(6)) / math.sqrt(len(g))
