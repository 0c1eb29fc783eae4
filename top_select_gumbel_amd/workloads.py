"""Seeded synthetic inputs for the sampling path (numpy PCG64; no method arithmetic here).

Both the oracle-side tests and the GPU side draw their inputs from this module, which
holds only data generation. All data is drawn in binary64 and cast to fp32; per-row
Philox seeds are drawn after the data.

Workloads (the sizes follow the pages' shapes; synthetic data stands in for the models
and prompts the pages measured on):

* ``tiny``        4 x 1024 N(0,1) logits, k=50, p=0.9, T=1; plus 200 rows of V=16.
* ``decode``      64 x 151936 logits 2.5*N(0,1) with 20 distinct head tokens raised by
                  +8 per row; k ~ U{1..1024}, p ~ U[0.5,1), T ~ U[0.5,1.5). V=151936 is the
                  vocabulary in RL-Kernel issue #332 ("Summary").
* ``decode_topp_only``  the decode rows with top-k disabled (k = V).
* ``heavy``       256 identical rows of V=32000, logits = log(counts), counts in {1,2,3}
                  and counts[0] = round(e^18) (vLLM PR #45996 summary, "key source
                  excerpts": the heavy-tailed fidelity test); k off, p=1, T=1.
* ``tie_stress``  128 x 128256 N(0,1)*1e5 rounded to the bf16 grid, the last row all
                  equal; k ~ U{1..2048}, p=0.95, T=1.
* ``indexer``     select only: 32 x 131072 keys N(0,1) rounded to 1e-3 (k=2048), one row of
                  1048576 such keys, one near-uniform row of 152000 keys (mlxcel issue #901,
                  "Task": the near-uniform 152K adversarial row).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

HEAVY_HEAD_COUNT = 65_659_969          # round(e^18)


@dataclass
class Batch:
    logits: np.ndarray                  # fp32 [B, V]
    k: Optional[np.ndarray] = None      # int32 [B]
    p: Optional[np.ndarray] = None      # fp32 [B]
    t: Optional[np.ndarray] = None      # fp32 [B]
    seeds: Optional[np.ndarray] = None  # uint64 [B]
    k_max: int = 0
    name: str = ""
    min_p: Optional[np.ndarray] = None  # fp32 [B]


def _seeds(rng, b):
    return rng.integers(0, 2 ** 64, size=b, dtype=np.uint64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even), returned as fp32."""
    bits = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def tiny(seed: int = 1) -> Batch:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, 1024)).astype(np.float32)
    return Batch(logits=x, k=np.full(4, 50, np.int32), p=np.full(4, 0.9, np.float32),
                 t=np.ones(4, np.float32), seeds=_seeds(rng, 4), k_max=50, name="tiny")


def tiny_v16(seed: int = 11, rows: int = 200) -> Batch:
    """Rows of V=16: half N(0,1), half small integers in {-2..2} (many exact ties)."""
    rng = np.random.default_rng(seed)
    half = rows // 2
    a = rng.standard_normal((half, 16))
    b = rng.integers(-2, 3, size=(rows - half, 16)).astype(np.float64)
    x = np.concatenate([a, b]).astype(np.float32)
    k = rng.integers(1, 17, size=rows).astype(np.int32)
    p = rng.uniform(0.0, 1.0, size=rows)
    p = np.where(p == 0.0, 1.0, p)
    p[rng.random(rows) < 0.1] = 1.0
    t = rng.uniform(0.25, 2.0, size=rows)
    t[rng.random(rows) < 0.1] = 0.0
    return Batch(logits=x, k=k, p=p.astype(np.float32), t=t.astype(np.float32),
                 seeds=_seeds(rng, rows), k_max=16, name="tiny_v16")


def decode(seed: int = 2, rows: int = 64, vocab: int = 151936) -> Batch:
    rng = np.random.default_rng(seed)
    x = 2.5 * rng.standard_normal((rows, vocab))
    for r in range(rows):
        head = rng.choice(vocab, 20, replace=False)
        x[r, head] += 8.0
    x = x.astype(np.float32)
    k = rng.integers(1, 1025, size=rows).astype(np.int32)
    p = rng.uniform(0.5, 1.0, size=rows).astype(np.float32)
    t = rng.uniform(0.5, 1.5, size=rows).astype(np.float32)
    return Batch(logits=x, k=k, p=p, t=t, seeds=_seeds(rng, rows), k_max=1024, name="decode")


def decode_topp_only(seed: int = 2, rows: int = 64, vocab: int = 151936) -> Batch:
    """The decode rows with top-k disabled (k = V): top-p over the whole row."""
    b = decode(seed, rows, vocab)
    b.k = np.full(rows, vocab, np.int32)
    b.k_max = vocab
    b.name = "decode_topp_only"
    return b


def heavy_counts(seed: int = 3, vocab: int = 32000) -> np.ndarray:
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, 4, size=vocab).astype(np.int64)
    counts[0] = HEAVY_HEAD_COUNT
    return counts


def heavy(seed: int = 3, rows: int = 256, vocab: int = 32000) -> Batch:
    counts = heavy_counts(seed, vocab)
    row = np.log(counts.astype(np.float64)).astype(np.float32)
    x = np.tile(row, (rows, 1))
    return Batch(logits=x, k=np.full(rows, vocab, np.int32), p=np.ones(rows, np.float32),
                 t=np.ones(rows, np.float32), seeds=None, k_max=vocab, name="heavy")


def heavy_launch_seeds(j: int, rows: int = 256) -> np.ndarray:
    """Launch j of the heavy-tailed test uses one seed for all rows (rows differ by counter)."""
    return np.full(rows, 0x5EED0000 + j, np.uint64)


def tie_stress(seed: int = 4, rows: int = 128, vocab: int = 128256) -> Batch:
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows - 1, vocab)) * 1e5).astype(np.float32)
    x = bf16_round(x)
    flat = np.full((1, vocab), bf16_round(np.float32(1e5)), np.float32)
    x = np.concatenate([x, flat]).astype(np.float32)
    k = rng.integers(1, 2049, size=rows).astype(np.int32)
    return Batch(logits=x, k=k, p=np.full(rows, 0.95, np.float32), t=np.ones(rows, np.float32),
                 seeds=_seeds(rng, rows), k_max=2048, name="tie_stress")


def indexer_rows(seed: int = 5, rows: int = 32, n: int = 131072) -> Batch:
    rng = np.random.default_rng(seed)
    x = np.round(rng.standard_normal((rows, n)), 3).astype(np.float32)
    return Batch(logits=x, k=np.full(rows, 2048, np.int32), k_max=2048, name=f"indexer_{rows}x{n}")


def indexer_long(seed: int = 6, n: int = 1048576) -> Batch:
    return indexer_rows(seed, 1, n)


def indexer_near_uniform(seed: int = 7, n: int = 152000) -> Batch:
    rng = np.random.default_rng(seed)
    x = (1.0 + 1e-6 * rng.standard_normal((1, n))).astype(np.float32)
    return Batch(logits=x, k=np.full(1, 2048, np.int32), k_max=2048, name="indexer_near_uniform")


def small_random(seed: int, rows: int, vocab: int, k_hi: int, *, scale: float = 1.0,
                 tie_levels: int = 0, p_lo: float = 0.5) -> Batch:
    """General small batches for parity sweeps (optionally with heavy exact ties)."""
    rng = np.random.default_rng(seed)
    if tie_levels:
        x = rng.integers(0, tie_levels, size=(rows, vocab)).astype(np.float64) * scale
    else:
        x = rng.standard_normal((rows, vocab)) * scale
    x = x.astype(np.float32)
    k = rng.integers(1, k_hi + 1, size=rows).astype(np.int32)
    p = rng.uniform(p_lo, 1.0, size=rows).astype(np.float32)
    t = rng.uniform(0.5, 1.5, size=rows).astype(np.float32)
    return Batch(logits=x, k=k, p=p, t=t, seeds=_seeds(rng, rows), k_max=int(k_hi),
                 name=f"random_{rows}x{vocab}")


def rejection_mix(seed: int, rows: int, vocab: int, *, tie_levels: int = 0, masked: float = 0.0) -> Batch:
    """Parameter mix for the rejection sampler: top-k only, top-p only, joint, min-p, off and
    greedy rows (mlxcel issue #901, "Performance validation": top-k 40, top-p 0.9, min-p
    0.05 and top-k + top-p); optional exact ties and -inf (masked) tokens."""
    rng = np.random.default_rng(seed)
    if tie_levels:
        x = rng.integers(0, tie_levels, size=(rows, vocab)).astype(np.float64)
    else:
        x = rng.standard_normal((rows, vocab)) * 2.0
    if masked:
        x[rng.random((rows, vocab)) < masked] = -np.inf
    x = x.astype(np.float32)
    kind = np.arange(rows) % 6
    k = np.where((kind == 0) | (kind == 2), rng.integers(1, 200, size=rows), vocab + 5).astype(np.int32)
    p = np.where((kind == 1) | (kind == 2), rng.uniform(0.3, 1.0, size=rows), 1.0).astype(np.float32)
    mp = np.where(kind == 3, rng.uniform(0.01, 0.3, size=rows), 0.0).astype(np.float32)
    t = rng.uniform(0.5, 1.5, size=rows)
    t[kind == 5] = 0.0
    return Batch(logits=x, k=k, p=p, t=t.astype(np.float32), seeds=_seeds(rng, rows),
                 name=f"rejection_{rows}x{vocab}", min_p=mp)
