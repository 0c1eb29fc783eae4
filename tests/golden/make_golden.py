"""Writes the stored expectations of the pooled statistical GPU tests. Calls only oracle/.

  decode_topp_pooled.txt  top-p kept counts of 1024 decode rows (the decode workload at
                          seeds 2 + 100*j, j < 16): the count-equality rule is judged on a pool
                          of at least 1000 rows, which one 64-row batch cannot give.
  heavy_first_draws.txt   the sampled token and score gap of the first 2048 draws of the
                          heavy-tailed fidelity test (launch j uses one seed for all 256 rows).

Run from the repository root: python tests/golden/make_golden.py  (about a minute on 8 cores)
"""
import multiprocessing as mp
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from top_select_gumbel_amd import workloads as wl  # noqa: E402

DECODE_SEEDS = [2 + 100 * j for j in range(16)]
HEAVY_LAUNCHES = 8


def decode_rows(seed):
    b = wl.decode(seed)
    out = []
    for r in range(b.logits.shape[0]):
        res = oracle.topp_row(b.logits[r], int(b.k[r]), oracle.to_f32(b.p[r]), oracle.to_f32(b.t[r]))
        out.append((seed, r, res.status, res.kept, int(res.ambiguous)))
    return out


def heavy_draws(j):
    b = wl.heavy()
    seeds = wl.heavy_launch_seeds(j)
    out = []
    for r in range(b.logits.shape[0]):
        res = oracle.sample_row(b.logits[r], None, 1.0, 1.0, int(seeds[r]), r)
        out.append((j, r, res.token, res.gap))
    return out


def main():
    with mp.Pool(min(8, os.cpu_count() or 1)) as pool:
        dec = [row for part in pool.map(decode_rows, DECODE_SEEDS) for row in part]
        hv = [row for part in pool.map(heavy_draws, range(HEAVY_LAUNCHES)) for row in part]
    with open(os.path.join(HERE, "decode_topp_pooled.txt"), "w") as f:
        f.write("# oracle top-p of the decode workload (k ~ U{1..1024}, p ~ U[0.5,1), T ~ U[0.5,1.5)),\n")
        f.write("# seeds 2 + 100*j for j < 16; written by tests/golden/make_golden.py (oracle only)\n")
        f.write("# seed row status kept ambiguous\n")
        for seed, r, st, kept, amb in dec:
            f.write(f"{seed} {r} {st} {kept} {amb}\n")
    with open(os.path.join(HERE, "heavy_first_draws.txt"), "w") as f:
        f.write("# oracle draws of the heavy-tailed fidelity test (vLLM PR #45996 summary, \"key source excerpts\"):\n")
        f.write("# 256 rows of log(counts), V=32000, k off, p=1, T=1;\n")
        f.write("# launch j uses seed 0x5EED0000 + j for every row; written by tests/golden/make_golden.py\n")
        f.write("# launch row token gap\n")
        for j, r, tok, gap in hv:
            f.write(f"{j} {r} {tok} {gap!r}\n")


if __name__ == "__main__":
    main()
