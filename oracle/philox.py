"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE ONLY: this module belongs to the CPU oracle. Only tests/,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The GPU library carries its own, separately written Philox.

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11 (the Philox-4x32 bijection with R = 10
rounds). The sampling pages name only "a counter-based Philox4x32-10 stream
keyed by (seed, row, token)"; the word layout below is this library's reading
of that phrase:

* key      = (seed mod 2^32, seed div 2^32)            two 32-bit words
* counter  = (token div 4, row, 0, 0)                   four 32-bit words
* the word used for ``token`` is output word ``token mod 4``.

One round maps the counter (c0, c1, c2, c3) under key (k0, k1) to
(hi(B*c2) ^ c1 ^ k0, lo(B*c2), hi(A*c0) ^ c3 ^ k1, lo(A*c0)) with the two
round multipliers A = 0xD2511F53 and B = 0xCD9E8D57 (hi/lo: upper/lower 32 bits
of the 64-bit product). Between rounds the key is advanced by the Weyl
constants (0x9E3779B9, 0xBB67AE85), modulo 2^32.
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
MUL_A = 0xD2511F53
MUL_B = 0xCD9E8D57
WEYL_0 = 0x9E3779B9
WEYL_1 = 0xBB67AE85
ROUNDS = 10


def philox4x32(ctr, key, rounds: int = ROUNDS):
    """One Philox4x32 block on Python ints: returns four 32-bit output words."""
    c0, c1, c2, c3 = (int(v) & MASK32 for v in ctr)
    k0, k1 = (int(v) & MASK32 for v in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + WEYL_0) & MASK32
            k1 = (k1 + WEYL_1) & MASK32
        prod_a = MUL_A * c0
        prod_b = MUL_B * c2
        c0, c1, c2, c3 = (
            (prod_b >> 32) ^ c1 ^ k0,
            prod_b & MASK32,
            (prod_a >> 32) ^ c3 ^ k1,
            prod_a & MASK32,
        )
    return c0, c1, c2, c3


def philox4x32_np(c0, c1, c2, c3, k0: int, k1: int, rounds: int = ROUNDS):
    """Vectorised Philox4x32 over arrays of counters (uint64 arithmetic in numpy).

    Same map as :func:`philox4x32`; every product of two 32-bit words fits in 64
    bits, so uint64 holds it exactly.
    """
    m = np.uint64(MASK32)
    c = [np.asarray(v, dtype=np.uint64) & m for v in (c0, c1, c2, c3)]
    shape = np.broadcast(*c).shape
    c = [np.broadcast_to(v, shape).copy() for v in c]
    k0 = np.uint64(k0 & MASK32)
    k1 = np.uint64(k1 & MASK32)
    a = np.uint64(MUL_A)
    b = np.uint64(MUL_B)
    for r in range(rounds):
        if r:
            k0 = (k0 + np.uint64(WEYL_0)) & m
            k1 = (k1 + np.uint64(WEYL_1)) & m
        prod_a = a * c[0]
        prod_b = b * c[2]
        c = [
            (prod_b >> np.uint64(32)) ^ c[1] ^ k0,
            prod_b & m,
            (prod_a >> np.uint64(32)) ^ c[3] ^ k1,
            prod_a & m,
        ]
    return tuple(v.astype(np.uint32) for v in c)


def seed_key(seed: int):
    """Split a 64-bit per-row seed into the two Philox key words (low, high)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & MASK32, seed >> 32


def token_words(seed: int, row: int, tokens) -> np.ndarray:
    """The 32-bit random word for each token id in ``tokens`` of row ``row``."""
    toks = np.asarray(tokens, dtype=np.int64)
    k0, k1 = seed_key(seed)
    words = philox4x32_np(toks >> 2, np.full_like(toks, int(row) & MASK32), 0, 0, k0, k1)
    lane = toks & 3
    out = np.empty(toks.shape, dtype=np.uint32)
    for j in range(4):
        sel = lane == j
        out[sel] = words[j][sel]
    return out
