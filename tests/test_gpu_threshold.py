"""GPU parity on rows whose candidate threshold is not found in the window below the sample
maximum.

The stream kernel places each chunk's candidate threshold from a sample: first in 256 bins of
2^16 keys reaching down from the sample maximum (about two binades), else by a two-level
search over the whole key range, refined through the low key bits when one bin holds many
sampled keys. These rows force the second search and the refinement: an outlier far above
the rest of the row inside the sampled slots, all-negative rows (log-probabilities: the keys
of the top tokens sit many binades apart in key space), magnitudes spread over forty
binades, and near-uniform rows. Every case prints a [case] line first.
"""
import numpy as np
import pytest

import top_select_gumbel_amd as ts
from gpu_helpers import banner, check_samples, check_topk, check_topp, dev, host, torch_cuda

pytestmark = pytest.mark.gpu

V = 40000   # five chunks per row, the last one ragged


def _rows(seed: int, rows: int = 8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, V))
    # 0-1: one outlier per chunk at the start of a chunk (inside the first wave's sampled slots)
    x[0, ::8000] = 1.0e6
    x[1, 3::8000] = 3.0e4
    # 2-3: log-probabilities (all negative, top tokens close to 0)
    x[2] = -np.abs(rng.standard_normal(V) * 4.0) - 1e-3
    x[3] = -rng.exponential(6.0, V) - 0.5
    # 4: magnitudes spread over forty binades, both signs
    x[4] = np.sign(rng.standard_normal(V)) * np.exp2(rng.uniform(-20.0, 20.0, V))
    # 5: near-uniform (every sampled key in one window bin: refined)
    x[5] = 1.0 + 1e-6 * rng.standard_normal(V)
    # 6: a bf16-grid tie row shifted far negative
    x[6] = np.round(rng.standard_normal(V) * 8.0) - 1.0e4
    # 7: one outlier per chunk that is the only value above a huge gap, plus a dense low band
    x[7] = rng.uniform(-1.0, 0.0, V)
    x[7, 5::8000] = 5.0e3
    x = x.astype(np.float32)
    k = rng.integers(1, 2049, size=rows).astype(np.int32)
    k[0] = 3
    p = rng.uniform(0.5, 1.0, size=rows).astype(np.float32)
    t = rng.uniform(0.5, 1.5, size=rows).astype(np.float32)
    seeds = rng.integers(0, 2 ** 64, rows, dtype=np.uint64)
    return x, k, p, t, seeds


@pytest.mark.parametrize("seed", [1, 2])
def test_threshold_fallback_rows_topk(seed):
    torch = torch_cuda()
    x, k, _, _, _ = _rows(seed)
    banner(f"threshold fallback rows: topk seed={seed} V={V}")
    out, st = ts.ts_topk_select(dev(x), dev(k), 2048)
    torch.cuda.synchronize()
    check_topk(x, k, 2048, host(out), host(st), f"fallback topk {seed}")


@pytest.mark.parametrize("seed", [1, 2])
def test_threshold_fallback_rows_topp_and_sample(seed):
    torch = torch_cuda()
    x, k, p, t, seeds = _rows(seed)
    banner(f"threshold fallback rows: topp seed={seed} V={V}")
    kept, mask, st = ts.ts_topp_mask(dev(x), dev(k), dev(p), dev(t), True)
    torch.cuda.synchronize()
    kept, mask, st = host(kept), host(mask), host(st)
    check_topp(x, k, p, t, kept, mask, st, f"fallback topp {seed}")
    banner(f"threshold fallback rows: sample seed={seed} V={V}")
    tok, st2 = ts.ts_sample_rows(dev(x), dev(k), dev(p), dev(t), dev(seeds))
    torch.cuda.synchronize()
    check_samples(x, k, p, t, seeds, host(tok), host(st2), kept, f"fallback sample {seed}")
