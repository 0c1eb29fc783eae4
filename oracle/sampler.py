"""Binary64 CPU oracle for per-row top-k select, top-p nucleus and Gumbel-max sampling.

TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously-correct reference that the
HIP library is checked against. It shares no code with the library; only tests/,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.

Page citations use the page title and the section on that page:

* [TOPP]   "Split top-p numerical reference and conservative gate" (anvil-serving
           finding), sections "Source basis", "Independent binary64 numerical
           reference", "Predeclared gate", "Breakage probes".
* [GUMBEL] prhub summary of vLLM PR #45996 (log1p(-u) for fp32 Gumbel sampling),
           sections "implementation breakdown" and "key source excerpts".
* [DETK]   vLLM PR #55122 "[Kernel] Make persistent_topk deterministic", sections
           "Changes" and "Test plan".
* [LOGP]   RL-Kernel issue #332 "Deterministic SM90 linear_logp", sections
           "Design: the numeric contract" and "Integration".
* [REJ]    mlxcel issue #901 "Sorting-free top-k/top-p/min-p sampling with dual-pivot
           rejection kernels", sections "Task" and "Regression guard".

Readings taken where the pages are silent (each is listed with its reason in the
design notes of the repository):

* transform order is temperature -> top-k -> top-p -> sample ([LOGP] "Integration");
  the top-p normaliser is taken over the top-k set;
* ranking uses the raw fp32 logits; temperature enters only the exponent and the
  Gumbel score;
* p == 1.0 (after fp32 conversion) means "top-p off": all of the top-k set is kept;
* k >= V means "top-k off"; T == 0 means greedy (the canonical first token);
* NaN or +inf logits, or a row of only -inf, reject the row; -inf marks a masked
  token (weight 0, ranked last, never sampled). For top-k select only NaN rejects;
* status precedence when several checks fail: logits (1), k (2), p (3), T (4).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .philox import token_words

STATUS_OK = 0
STATUS_NONFINITE = 1
STATUS_BAD_K = 2
STATUS_BAD_P = 3
STATUS_BAD_T = 4
STATUS_BAD_MINP = 5

U_MIN = 2.0 ** -32          # smallest nonzero value of word * 2^-32
U_MAX = 1.0 - 2.0 ** -24    # largest fp32 below 1.0: keeps log1p(-u) finite


def to_f32(v) -> float:
    """Round a number to the nearest fp32 value and return it as a Python float."""
    return float(np.float32(v))


def row_floats(row) -> List[float]:
    """fp32 logits -> exact Python floats ([TOPP] reference step 1: keep the fp32 values)."""
    return np.asarray(row, dtype=np.float32).astype(np.float64).tolist()


# --------------------------------------------------------------------------- validation
def logits_status(x: Sequence[float], *, select_only: bool = False) -> int:
    """Status of the logits alone ([TOPP] "Breakage probes": non-finite inputs fail closed).

    For sampling/top-p: NaN or +inf anywhere, or no finite-or-(-inf)-above-(-inf) token,
    rejects the row. For select-only, +-inf are ordinary keys and only NaN rejects.
    """
    if any(math.isnan(v) for v in x):
        return STATUS_NONFINITE
    if select_only:
        return STATUS_OK
    if any(v == math.inf for v in x):
        return STATUS_NONFINITE
    if all(v == -math.inf for v in x):
        return STATUS_NONFINITE
    return STATUS_OK


def params_status(k: Optional[int], p: Optional[float], t: Optional[float]) -> int:
    """Per-row parameter checks: k >= 1; p in (0, 1] after fp32 cast; T finite and >= 0."""
    if k is not None and int(k) < 1:
        return STATUS_BAD_K
    if p is not None and not (p > 0.0 and p <= 1.0):   # NaN fails both comparisons
        return STATUS_BAD_P
    if t is not None and (math.isnan(t) or math.isinf(t) or t < 0.0):
        return STATUS_BAD_T
    return STATUS_OK


# --------------------------------------------------------------------------- ordering
def canonical_order(x: Sequence[float]) -> List[int]:
    """Token ids sorted by (logit descending, token id ascending).

    [TOPP] reference step 2 (stable sort, token-id tie rule) and [DETK] "Changes"
    (top-k equals value-descending / index-ascending). Python treats -0.0 == 0.0,
    so signed zeros tie and fall back to the index, as [DETK] canonicalises them.
    """
    return sorted(range(len(x)), key=lambda i: (-x[i], i))


# --------------------------------------------------------------------------- top-k select
def topk_select_row(row, k: int, k_max: int):
    """Top-k select of one row: (status, out_idx list of length k_max).

    [DETK] "Changes": the output is the top-k by value desc / index asc, emitted in
    ascending index order; unused slots are -1 (short rows, "Test plan").
    """
    x = row_floats(row)
    st = logits_status(x, select_only=True)
    if st == STATUS_OK and int(k) < 1:
        st = STATUS_BAD_K
    ke = min(int(k), len(x)) if st == STATUS_OK else 0
    if st == STATUS_OK and ke > k_max:
        st = STATUS_BAD_K
    if st != STATUS_OK:
        return st, [-1] * k_max
    chosen = sorted(canonical_order(x)[:ke])
    return STATUS_OK, chosen + [-1] * (k_max - ke)


ORDER_INDEX = 0
ORDER_VALUE = 1


def topk_select_rows_row(row, length: Optional[int], k: int, k_max: int, order: int = ORDER_INDEX,
                         offset: int = 0):
    """Top-k of a row's valid prefix, for sparse-indexer rows of varying length.

    [DETK] "Changes" (filtered-row length clamping) and "Test plan" (short rows padded with
    -1): only keys [0, n) take part, n = length clamped to [0, len(row)] (None = the whole
    row); a NaN there rejects the row (one past n does not). The selection is the first
    min(k, n) ids of the canonical order of that prefix. Output order: ascending id
    (ORDER_INDEX, as [DETK] emits) or the canonical order itself (ORDER_VALUE: value
    descending, id ascending, as a value-ordered top-k returns it). Each emitted id is
    shifted by ``offset`` (the row's start in a ragged index space); unused slots are -1.
    """
    x = row_floats(row)
    n = len(x) if length is None else max(0, min(int(length), len(x)))
    x = x[:n]
    st = logits_status(x, select_only=True) if n > 0 else STATUS_OK
    if st == STATUS_OK and int(k) < 1:
        st = STATUS_BAD_K
    ke = min(int(k), n) if st == STATUS_OK else 0
    if st == STATUS_OK and ke > k_max:
        st = STATUS_BAD_K
    if st != STATUS_OK:
        return st, [-1] * k_max
    chosen = canonical_order(x)[:ke]
    if order == ORDER_INDEX:
        chosen = sorted(chosen)
    return STATUS_OK, [offset + i for i in chosen] + [-1] * (k_max - ke)


def topk_select_rows(x2d, lengths, k, k_max: int, order: int = ORDER_INDEX, offsets=None):
    """Batched form of topk_select_rows_row: (status[B], out_idx[B, k_max]) int32 arrays."""
    x2d = np.asarray(x2d, dtype=np.float32)
    b = x2d.shape[0]
    status = np.zeros(b, np.int32)
    out = np.full((b, k_max), -1, np.int64)
    for r in range(b):
        st, idx = topk_select_rows_row(x2d[r], None if lengths is None else int(lengths[r]), int(k[r]), k_max,
                                       order, 0 if offsets is None else int(offsets[r]))
        status[r] = st
        out[r] = idx
    return status, out.astype(np.int32)


# --------------------------------------------------------------------------- top-p
@dataclass
class ToppResult:
    status: int
    kept: int = 0                       # |P|
    order: List[int] = field(default_factory=list)   # canonical order of the row
    topk: List[int] = field(default_factory=list)    # K, canonical order
    kept_ids: List[int] = field(default_factory=list)  # P, canonical order (a prefix of K)
    weights: List[float] = field(default_factory=list)  # w over K, canonical order
    z: float = 0.0
    target: float = 0.0
    ambiguous: bool = False             # oracle_boundary_ambiguous ([TOPP] step 6)
    minp_ambiguous: bool = False        # a kept weight within 1e-6 of min_p
    m: float = 0.0                      # row maximum logit
    x: List[float] = field(default_factory=list)


def neumaier_first_reach(w: Sequence[float], target: float) -> int:
    """Smallest n whose compensated prefix sum of w[:n] reaches target ([TOPP] step 5)."""
    s = 0.0
    c = 0.0
    for j, v in enumerate(w):
        t = s + v
        if abs(s) >= abs(v):
            c += (s - t) + v
        else:
            c += (v - t) + s
        s = t
        if s + c >= target:
            return j + 1
    return len(w)


def topp_row(row, k: Optional[int], p: Optional[float], t: Optional[float]) -> ToppResult:
    """Top-k then top-p over one row, in binary64 ([TOPP] "Independent binary64 numerical reference").

    k, p, t are the per-row values after fp32 conversion (None = the op's default:
    top-k off, p = 1, T = 1).
    """
    x = row_floats(row)
    pv = 1.0 if p is None else float(p)
    tv = 1.0 if t is None else float(t)
    st = logits_status(x)
    if st == STATUS_OK:
        st = params_status(k, pv, tv)
    if st != STATUS_OK:
        return ToppResult(status=st, x=x)
    order = canonical_order(x)
    ke = len(x) if k is None else min(int(k), len(x))
    topk = order[:ke]
    m = x[order[0]]
    res = ToppResult(status=STATUS_OK, order=order, topk=topk, m=m, x=x)
    if tv == 0.0:                       # greedy: the canonical first token only
        res.kept = 1
        res.kept_ids = [order[0]]
        return res
    # [TOPP] step 3: subtract the maximum, binary64 exp; temperature in the exponent.
    w = [math.exp((x[i] - m) / tv) for i in topk]
    res.weights = w
    if pv == 1.0:                       # top-p off: keep all of K, no arithmetic
        res.kept = ke
        res.kept_ids = list(topk)
        res.z = math.fsum(w)
        res.target = res.z
        return res
    z = math.fsum(w)                    # [TOPP] step 4
    target = pv * z
    n = neumaier_first_reach(w, target)  # [TOPP] step 5
    hi_ok = math.fsum(w[:n]) >= target
    lo_ok = n == 1 or math.fsum(w[: n - 1]) < target
    res.ambiguous = not (hi_ok and lo_ok)  # [TOPP] step 6
    res.z = z
    res.target = target
    res.kept = n
    res.kept_ids = topk[:n]
    return res


# --------------------------------------------------------------------------- Gumbel noise
def uniform_from_word(word: int) -> float:
    """u = fp32(word * 2^-32) clamped to [2^-32, 1 - 2^-24].

    [GUMBEL] "implementation breakdown": clamp u at the generator's true minimum
    (for word * 2^-32 that minimum is 2^-32); the upper clamp keeps log1p(-u) finite.
    """
    u = to_f32(int(word) * U_MIN)
    return min(max(u, U_MIN), U_MAX)


def gumbel_from_word(word: int) -> float:
    """Gumbel noise g = -log(-log1p(-u)) in binary64 ([GUMBEL] "key source excerpts")."""
    u = uniform_from_word(word)
    return -math.log(-math.log1p(-u))


def gumbel_noise(seed: int, row: int, tokens) -> List[float]:
    """Noise of each token of ``row`` under ``seed`` (Philox word, then the map above)."""
    return [gumbel_from_word(int(wd)) for wd in token_words(seed, row, tokens)]


# --------------------------------------------------------------------------- sampling
@dataclass
class SampleResult:
    status: int
    token: int = -1
    gap: float = math.inf               # best minus second-best perturbed score
    topp: Optional[ToppResult] = None


def gumbel_argmax(x: Sequence[float], m: float, t: float, kept: Sequence[int],
                  seed: int, row: int):
    """Argmax over ``kept`` of (x_i - m)/T + g_i, lowest id on exact ties; also the gap.

    [GUMBEL] "key source excerpts": add the noise to the (temperature-scaled) logits of
    the kept tokens and take the maximum with its index.
    """
    ids = sorted(kept)
    g = gumbel_noise(seed, row, ids)
    scores = [((x[i] - m) / t + gi, i) for i, gi in zip(ids, g)]
    best_s = max(s for s, _ in scores)
    best_i = min(i for s, i in scores if s == best_s)
    rest = [s for s, i in scores if i != best_i]
    if not rest:
        return best_i, math.inf
    return best_i, best_s - max(rest)


def sample_row(row, k: Optional[int], p: Optional[float], t: Optional[float],
               seed: int, row_index: int) -> SampleResult:
    """One sampled token id for one row: top-k, top-p, then Gumbel-max over the kept set."""
    tp = topp_row(row, k, p, t)
    if tp.status != STATUS_OK:
        return SampleResult(status=tp.status, topp=tp)
    tv = 1.0 if t is None else float(t)
    if tv == 0.0:
        return SampleResult(status=STATUS_OK, token=tp.order[0], gap=math.inf, topp=tp)
    tok, gap = gumbel_argmax(tp.x, tp.m, tv, tp.kept_ids, seed, row_index)
    return SampleResult(status=STATUS_OK, token=tok, gap=gap, topp=tp)


def lse_logp_row(row, t: Optional[float], token: int):
    """Temperature-scaled log-sum-exp of a whole row and the log-probability of ``token``.

    [LOGP] "Design: the numeric contract": m = max of the row, S = sum of exp(x - m),
    lse = m + log S, logp = min(x_t - lse, 0); temperature enters in the epilogue
    ([LOGP] "Contract constants", temperature), so with x/T in place of x:
    lse = m/T + log(sum exp((x - m)/T)) and logp = min(x_t/T - lse, 0). The sum is over the
    whole row (the model's distribution at temperature T), in binary64 with math.fsum;
    -inf logits contribute 0. T == 0 (greedy): lse = +inf and the greedy token has logp 0.
    """
    x = row_floats(row)
    tv = 1.0 if t is None else float(t)
    if tv == 0.0:
        return math.inf, 0.0
    m = max(x)
    s = math.fsum(math.exp((xi - m) / tv) for xi in x if xi != -math.inf)
    lse = m / tv + math.log(s)
    return lse, min(x[token] / tv - lse, 0.0)


def sample_logp_rows(x2d, k, p, t, seeds):
    """Batched sampling with the selected token's logprob: list of
    (SampleResult, lse, logp), lse and logp for the oracle's own token (nan for rows
    that are rejected)."""
    x2d = np.asarray(x2d, dtype=np.float32)
    out = []
    for r, res in enumerate(sample_rows(x2d, k, p, t, seeds)):
        if res.status != STATUS_OK:
            out.append((res, math.nan, math.nan))
            continue
        lse, logp = lse_logp_row(x2d[r], _opt(t, r, to_f32), res.token)
        out.append((res, lse, logp))
    return out


MINP_AMBIGUOUS_REL = 1e-6


def minp_filter(res: ToppResult, min_p: Optional[float]) -> ToppResult:
    """min-p after top-p, the pinned transform order temperature -> top-k -> top-p -> min-p
    ([LOGP] relay program with pinned order; [REJ] "Task": min-p on probabilities).

    A token of P stays when its probability is at least min_p times the largest one:
    w_i / Z >= min_p * (1 / Z), i.e. w_i >= min_p with the binary64 weights of the top-p
    step (w = 1 for the row maximum, which therefore always stays). Weights fall along the
    canonical order, so the result is again a canonical prefix. min_p = 0 (or None) is off;
    min_p must lie in [0, 1] (else status 5, after the checks of the other parameters).
    ``minp_ambiguous`` marks rows where a weight of P lies within 1e-6 (relative) of min_p,
    where a result computed in another precision may legitimately differ.
    """
    if min_p is None or res.status != STATUS_OK:
        return res
    mp = float(min_p)
    if not (mp >= 0.0 and mp <= 1.0):
        return ToppResult(status=STATUS_BAD_MINP, x=res.x)
    if mp == 0.0 or not res.weights:     # off, or greedy (only the maximum is kept)
        return res
    w = res.weights
    n = 0
    while n < res.kept and w[n] >= mp:
        n += 1
    out = ToppResult(status=STATUS_OK, order=res.order, topk=res.topk, weights=res.weights,
                     z=res.z, target=res.target, ambiguous=res.ambiguous, m=res.m, x=res.x)
    out.kept = n
    out.kept_ids = res.kept_ids[:n]
    out.minp_ambiguous = any(abs(w[i] - mp) <= MINP_AMBIGUOUS_REL * mp for i in range(res.kept))
    return out


def topp_minp_row(row, k, p, t, min_p) -> ToppResult:
    """Top-k, top-p, then min-p over one row."""
    return minp_filter(topp_row(row, k, p, t), min_p)


def sample_minp_row(row, k, p, t, min_p, seed: int, row_index: int) -> SampleResult:
    """One sampled token id for one row after top-k, top-p and min-p."""
    tp = topp_minp_row(row, k, p, t, min_p)
    if tp.status != STATUS_OK:
        return SampleResult(status=tp.status, topp=tp)
    tv = 1.0 if t is None else float(t)
    if tv == 0.0:
        return SampleResult(status=STATUS_OK, token=tp.order[0], gap=math.inf, topp=tp)
    tok, gap = gumbel_argmax(tp.x, tp.m, tv, tp.kept_ids, seed, row_index)
    return SampleResult(status=STATUS_OK, token=tok, gap=gap, topp=tp)


# --------------------------------------------------------------------------- batched
def _opt(arr, r, cast):
    return None if arr is None else cast(arr[r])


def topk_select(x2d, k, k_max: int):
    """Batched top-k select: (status[B], out_idx[B, k_max]) as numpy int32 arrays."""
    x2d = np.asarray(x2d, dtype=np.float32)
    b = x2d.shape[0]
    status = np.zeros(b, np.int32)
    out = np.full((b, k_max), -1, np.int32)
    for r in range(b):
        st, idx = topk_select_row(x2d[r], int(k[r]), k_max)
        status[r] = st
        out[r] = idx
    return status, out


def topp_mask(x2d, k=None, p=None, t=None):
    """Batched top-p: list of ToppResult, one per row."""
    x2d = np.asarray(x2d, dtype=np.float32)
    return [topp_row(x2d[r], _opt(k, r, int), _opt(p, r, to_f32), _opt(t, r, to_f32))
            for r in range(x2d.shape[0])]


def sample_rows(x2d, k, p, t, seeds):
    """Batched sampling: list of SampleResult, one per row (row index = Philox row word)."""
    x2d = np.asarray(x2d, dtype=np.float32)
    return [sample_row(x2d[r], _opt(k, r, int), _opt(p, r, to_f32), _opt(t, r, to_f32),
                       int(seeds[r]), r)
            for r in range(x2d.shape[0])]


def topp_minp_mask(x2d, k, p, t, min_p):
    """Batched top-k / top-p / min-p: list of ToppResult, one per row."""
    x2d = np.asarray(x2d, dtype=np.float32)
    return [topp_minp_row(x2d[r], _opt(k, r, int), _opt(p, r, to_f32), _opt(t, r, to_f32),
                          _opt(min_p, r, to_f32))
            for r in range(x2d.shape[0])]


def sample_rows_minp(x2d, k, p, t, min_p, seeds):
    """Batched sampling after top-k / top-p / min-p (row index = Philox row word)."""
    x2d = np.asarray(x2d, dtype=np.float32)
    return [sample_minp_row(x2d[r], _opt(k, r, int), _opt(p, r, to_f32), _opt(t, r, to_f32),
                            _opt(min_p, r, to_f32), int(seeds[r]), r)
            for r in range(x2d.shape[0])]
