"""The allocation-free entry point, ts_sample_rows_noalloc, called through the C ABI.

For callers that cannot allocate (graph capture, tight serving loops): its kernels keep
their workspace in the library's static device scratch. Its results must equal those of
ts_sample_rows (which takes a caller workspace) byte for byte, on two calls in a row on the
same GPU, the second with a smaller batch, so the second call runs over the first one's
leftovers in the shared scratch. Both batches include tie-heavy rows whose waves publish more
candidates than the allocation-free slices hold, so those rows take the exact path there, and
rows whose top-k entry reaches the vocabulary, which take the split nucleus (its parts' slots
live in the candidate area, so the smaller allocation-free slices give the second batch fewer
parts per row: 3 against 8, and hold no per-token bin codes beside them: there the cut bin's
tokens come from the row's values, against the codes of the workspace entry point).
"""
import ctypes

import numpy as np
import pytest

import top_select_gumbel_amd as ts
from top_select_gumbel_amd import workloads as wl
from gpu_helpers import banner, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


def batch(rows, vocab, seed):
    b = wl.decode(seed, rows, vocab)
    x = b.logits.copy()
    x[1] = np.float32(2.5)                             # all equal: every wave overflows
    x[2, : vocab // 2] = np.float32(7.0)               # half the row tied at the top
    k = b.k.copy()
    k[1], k[2] = 700, 1500
    k[3], k[4] = vocab, vocab + 5                      # top-k off by value: the split nucleus,
    p = b.p.copy()                                     # over as many parts as each scratch holds
    p[4] = np.float32(0.3)
    return x, k, p, b.t, b.seeds


def run_both(x, k, p, t, seeds):
    torch = torch_cuda()
    lib = ts.load_library()
    rows, vocab = x.shape
    xd, kd, pd, td = dev(x), dev(k), dev(p), dev(t)
    sd = dev(np.asarray(seeds, np.uint64))
    tok_ws, st_ws = ts.ts_sample_rows(xd, kd, pd, td, sd)
    tok = torch.full((rows,), -7, dtype=torch.int32, device="cuda:0")
    st = torch.full((rows,), -7, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.ts_sample_rows_noalloc(xd.data_ptr(), rows, vocab, vocab, kd.data_ptr(), pd.data_ptr(),
                                    td.data_ptr(), sd.data_ptr(), tok.data_ptr(), st.data_ptr(), stream)
    assert rc == 0, lib.ts_last_error().decode()
    torch.cuda.synchronize()
    return host(tok_ws), host(st_ws), host(tok), host(st)


def test_noalloc_matches_workspace_entry_point_twice():
    banner("noalloc: decode 64x151936, then 24x50000, against ts_sample_rows")
    for rows, vocab, seed in ((64, 151936, 2), (24, 50000, 5)):
        x, k, p, t, seeds = batch(rows, vocab, seed)
        tok_ws, st_ws, tok, st = run_both(x, k, p, t, seeds)
        assert np.array_equal(st, st_ws) and not st.any()
        assert np.array_equal(tok, tok_ws), f"{rows}x{vocab}: rows {np.nonzero(tok != tok_ws)[0][:8]}"
        assert tok[1] < k[1] and x[2, tok[2]] >= np.float32(7.0)   # tie rows: inside their top-k


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    lib = ts.load_library()
    fake = ctypes.c_void_p(0x1000)                      # never dereferenced: rejected first
    rc = lib.ts_sample_rows_noalloc(fake, 4096, 151936, 151936, None, None, None, fake, fake, None, None)
    assert rc == ts.TS_ERR_INVALID_ARG
    assert "scratch" in lib.ts_last_error().decode()
