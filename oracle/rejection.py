"""Binary64 CPU oracle for dual-pivot rejection sampling (a sorting-free sampler).

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by tests/,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``, never by the
library. It shares no code with the HIP library.

Source: [REJ] mlxcel issue #901 "Sorting-free top-k/top-p/min-p sampling with dual-pivot
rejection kernels": section "Background" (the per-filter algorithms: one candidate per
round from a CDF scan restricted to the entries above the lower bound, a second pivot
halfway between the candidate and the upper bound, counts and masses above both pivots,
accept or shrink the interval and renormalise; min-p as one filter on the row maximum;
the joint top-k + top-p loop with both accept tests), section "Task" item 2 (a cap on the
rounds with an exact fallback for the row) and section "Regression guard" (the support
must equal the filters' sets with the token-id tie rule; same seed, same stream).

Readings where the page leaves a step open (listed with their reasons in the design notes):

* Support. With w_i = exp((x_i - m) / T) and the canonical order sigma (logit descending,
  id ascending), the support is the canonical prefix sigma[0:n_S],
  n_S = min(k, n_p, n_m): n_p is the shortest prefix whose mass reaches p * Z with Z the
  mass of the WHOLE row (the joint filter tests both conditions against the full
  distribution, the one form a single rejection loop can test), n_m counts the tokens
  with w >= min_p. p == 1 is top-p off, k >= V top-k off, min_p == 0 min-p off, T == 0
  greedy. The draw is P(i) proportional to w_i on the support.
* Mass. Each weight counts as the integer M_i = floor(w_i * 2^S), S = 63 - bitlen(V),
  so every sum is exact and independent of its order ([REJ] "Background", determinism
  option: a fixed-order scan). The top-p target is ceil(p * Z) exactly.
* Ranks and ties. "Entries greater than a pivot" compare logits, with equal logits ordered
  by id, so the accept test "fewer than k above the candidate" is the candidate's
  canonical rank and the support keeps the lowest ids among equal logits.
* Second pivot. Halfway between the candidate's probability and the upper bound of the
  interval, in probability space ([REJ] "Background", top-k step (b)). Probabilities are the
  weights over Z, so the midpoint is taken on the weights: w1 = (w_c + w_hi) / 2 in binary64,
  with w_hi = 1 (the maximum's weight) at the start; "entries greater than the pivot" are the
  tokens with w > w1. When the support lies between the two pivots the upper bound becomes
  w1; when it lies above the second pivot the bound stays.
* Random words. Round j draws the 32-bit word 0 of Philox4x32-10 with key (seed lo, seed
  hi) and counter (j, row, 1, 0) (the Gumbel stream uses counter word 2 = 0); the CDF
  target is t = floor(word * Q / 2^32) for the current eligible mass Q, and the candidate
  is the first eligible id whose inclusive prefix mass exceeds t.
* Cap. After ``max_rounds`` rejected rounds the row falls back to one exact draw over the
  support (word of counter (max_rounds, row, 1, 0)); ``rounds`` reports -1 then.

Ambiguity: the GPU's weights carry about 1.6e-7 relative error. A row is flagged
``ambiguous`` when a CDF crossing, a top-p comparison, a min-p test or a token's weight
against the second pivot lies within that error of flipping; such rows are checked for
validity only. ``support_exact`` says whether the support's size itself is beyond doubt
(its boundary is set by k, or the top-p and min-p tests at the boundary are not close).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction
from typing import Callable, Optional

import numpy as np

from .philox import philox4x32, seed_key
from .sampler import (STATUS_BAD_MINP, STATUS_OK, logits_status, params_status, row_floats,
                      to_f32)

REL_ERR = 5e-7          # margin for the GPU's weight error (about 1.6e-7) plus rounding
MINP_REL = 1e-6         # min-p tests this close to a weight are flagged
PIVOT_REL = 1e-6        # weights this close to the second pivot are flagged
MAX_ROUNDS_LIMIT = 64


@dataclass
class RejectionResult:
    status: int
    token: int = -1
    rounds: int = 0            # accepted at this round (1-based); 0 greedy/rejected row; -1 fallback
    ambiguous: bool = False
    support_n: int = 0         # n_S by the definition
    support_exact: bool = True  # n_S is not within the weight error of a top-p / min-p flip
    order: Optional[np.ndarray] = None   # canonical order of the row


def _bitlen(n: int) -> int:
    return int(n).bit_length()


def round_word(seed: int, row: int, j: int) -> int:
    """The round-j random word of a row: Philox4x32-10 word 0 of counter (j, row, 1, 0)."""
    return philox4x32((j, row, 1, 0), seed_key(seed))[0]


def _canonical(x: np.ndarray) -> np.ndarray:
    """Canonical order (logit descending, id ascending); -0.0 and 0.0 tie."""
    ids = np.arange(x.shape[0])
    return np.lexsort((ids, -x))


def _above(x: np.ndarray, ids: np.ndarray, c: int) -> np.ndarray:
    """Entries ranked strictly above token c in the canonical order."""
    return (x > x[c]) | ((x == x[c]) & (ids < c))


def rejection_sample_row(row, k: Optional[int], p: Optional[float], t: Optional[float],
                         min_p: Optional[float], seed: int, row_index: int,
                         max_rounds: int = 32,
                         words: Optional[Callable[[int], int]] = None) -> RejectionResult:
    """One token of one row by dual-pivot rejection sampling ([REJ] "Background").

    ``words(j)`` overrides the round-j random word (tests drive worked examples with it).
    """
    word_of = words if words is not None else (lambda j: round_word(seed, row_index, j))
    x = np.asarray(row_floats(row), dtype=np.float64)
    V = x.shape[0]
    pv = 1.0 if p is None else float(p)
    tv = 1.0 if t is None else float(t)
    mp = 0.0 if min_p is None else float(min_p)
    st = logits_status(x.tolist())
    if st == STATUS_OK:
        st = params_status(k, pv, tv)
    if st == STATUS_OK and not (mp >= 0.0 and mp <= 1.0):
        st = STATUS_BAD_MINP
    if st != STATUS_OK:
        return RejectionResult(status=st)
    order = _canonical(x)
    if tv == 0.0:                                   # greedy: the canonical first token
        return RejectionResult(status=STATUS_OK, token=int(order[0]), rounds=0,
                               support_n=1, order=order)
    ids = np.arange(V)
    ke = V if k is None else min(int(k), V)
    m = float(x[order[0]])
    w = np.exp((x - m) / tv)                        # binary64; -inf -> 0
    S = 63 - _bitlen(V)
    M = np.floor(np.ldexp(w, S)).astype(np.int64)  # floor(w * 2^S), exact sums below 2^63
    Z = int(M.sum())
    topp_on = pv != 1.0
    target = math.ceil(Fraction(pv) * Z) if topp_on else None
    ok = (w >= mp) if mp > 0.0 else np.ones(V, dtype=bool)
    near_minp = (np.abs(w - mp) <= MINP_REL * mp) if mp > 0.0 else np.zeros(V, dtype=bool)

    # Support by its definition (for the fallback draw and for the tests).
    prefix = np.cumsum(M[order])
    n_p = int(np.searchsorted(prefix, target, side="left")) + 1 if topp_on else V
    n_m = int(ok.sum())
    n_s = min(ke, n_p, n_m)
    res = RejectionResult(status=STATUS_OK, support_n=n_s, order=order)

    def draw(eligible: np.ndarray, word: int) -> int:
        mass = np.where(eligible, M, 0)
        cum = np.cumsum(mass)
        q = int(cum[-1])
        tt = (word * q) >> 32
        c = int(np.searchsorted(cum, tt, side="right"))
        before = int(cum[c - 1]) if c > 0 else 0
        # A token near the min-p cut may be eligible on one side only: its mass widens the
        # margin the crossing must clear.
        delta = REL_ERR * q + 2 * int(eligible.sum()) + 2 + int(M[near_minp].sum())
        if (before > 0 and tt - before <= delta) or int(cum[c]) - 1 - tt < delta:
            res.ambiguous = True
        return c

    def near_target(mass: int) -> bool:
        return topp_on and abs(mass - target) <= REL_ERR * Z + 2 * V + 2

    eligible = ok.copy()
    hi = 1.0                                    # upper bound: the maximum's weight
    for j in range(max_rounds):
        c = draw(eligible, word_of(j))
        w1 = 0.5 * float(w[c]) + 0.5 * hi        # second pivot, halfway in probability
        above0 = _above(x, ids, c)
        n0 = int(above0.sum())
        mass0 = int(M[above0].sum())
        above1 = w > w1
        n1 = int(above1.sum())
        mass1 = int(M[above1].sum())
        if near_target(mass0) or near_target(mass1):
            res.ambiguous = True
        # A weight within the GPU's error of the pivot could land on the other side. Weights
        # of 1 (the maximum and its ties) are exact on both sides, and so is the pivot 1
        # (candidate of weight 1, bound 1), which no weight exceeds.
        if not (float(w[c]) == 1.0 and hi == 1.0):
            near = (np.abs(w - w1) <= PIVOT_REL * w1) & (w != 1.0)
            if bool(near.any()):
                res.ambiguous = True
        if n0 < ke and (not topp_on or mass0 < target):
            res.token = c
            res.rounds = j + 1
            break
        if n1 >= ke or (topp_on and mass1 >= target):
            eligible = above1 & ok              # the support lies above the second pivot
        else:
            eligible = above0 & ok              # the support lies above the candidate
            hi = w1
    else:
        res.rounds = -1
    # Is the support's size beyond the GPU's weight error? (It is exact when k sets it.)
    if n_s < ke:
        if topp_on and n_p == n_s:
            before = int(prefix[n_p - 2]) if n_p >= 2 else 0
            if near_target(int(prefix[n_p - 1])) or near_target(before):
                res.support_exact = False
        if mp > 0.0 and n_m == n_s and bool(near_minp.any()):
            res.support_exact = False
    if res.rounds != -1:
        return res
    # Cap reached: one exact draw over the support ([REJ] "Task" item 2).
    if not res.support_exact:
        res.ambiguous = True
    support = np.zeros(V, dtype=bool)
    support[order[:n_s]] = True
    res.token = draw(support, word_of(max_rounds))
    res.rounds = -1
    return res


def rejection_sample_rows(x2d, k, p, t, min_p, seeds, max_rounds: int = 32):
    """Batched rejection sampling: one RejectionResult per row (row index = Philox row word)."""
    x2d = np.asarray(x2d, dtype=np.float32)

    def opt(arr, r, cast):
        return None if arr is None else cast(arr[r])

    return [rejection_sample_row(x2d[r], opt(k, r, int), opt(p, r, to_f32), opt(t, r, to_f32),
                                 opt(min_p, r, to_f32), int(seeds[r]), r, max_rounds)
            for r in range(x2d.shape[0])]
