#!/usr/bin/env python3
"""Throughput of the batched sampling hot path on one MI355X.

One step = one ts_sample_rows call (top-k select, softmax + top-p cut, Gumbel-max sample)
over the decode workload: B=64 rows of V=151936 fp32 logits already resident in HBM.
Inputs rotate over enough distinct buffers (> 2x the 256 MB last-level cache) that every
step streams its logits from HBM ("cold"); a warm figure (same buffer every step) is
reported alongside.

Prints ONE JSON line (rank 0). Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
ROWS, VOCAB = 64, 151936
BYTES_PER_CALL = ROWS * VOCAB * 4
ROTATE = 16                    # 16 x 38.9 MB = 622 MB > 2 x 256 MB
SRC = os.path.join(ROOT, "top_select_gumbel_amd", "csrc")


# The sources of the two kernels of ts_sample_rows (the headline call); the rejection
# sampler's source is not part of it.
HEADLINE_SOURCES = ("topselect.hip", "ts_device.hpp")


def source_hash() -> str:
    h = hashlib.sha256()
    for name in HEADLINE_SOURCES:
        with open(os.path.join(SRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles():
    """HBM bytes per call from the committed PMC summary, if it was taken on the current kernels.

    The summary (a text file) holds `key: value` lines; `source_hash` must equal the hash of
    the kernel sources and `bytes_per_call` is FETCH_SIZE + WRITE_SIZE of the call's two
    kernels, scaled by the copy-kernel calibration factor.
    """
    path = os.path.join(ROOT, "profiles", "sample_rows_decode_traffic.txt")
    rec = {}
    try:
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith(("#", " ")):
                    k, v = line.split(":", 1)
                    rec[k.strip()] = v.strip()
    except OSError:
        return None
    if rec.get("source_hash") != source_hash():
        return None
    try:
        return float(rec["bytes_per_call"])
    except (KeyError, ValueError):
        return None


def _oracle_row(args):
    """One decode row through the oracle (a pool worker's unit of work)."""
    import oracle
    x, k, p, t, seed, r = args
    oracle.sample_row(x, k, p, t, seed, r)
    return r


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch, budget_s: float = 8.0):
    """Time the oracle (as it stands) on rows of the same workload: (i) one process on one
    host core, (ii) a process pool over rows. The pool has min(os.cpu_count(), 16) workers:
    16 cores is the host share of a one-GPU machine, whatever the count the container shows."""
    import multiprocessing as mp

    rows = batch.logits.shape[0]
    args = [(batch.logits[r], int(batch.k[r]), float(batch.p[r]), float(batch.t[r]), int(batch.seeds[r]), r)
            for r in range(rows)]
    t0 = time.perf_counter()
    n1 = 0
    while True:
        _oracle_row(args[n1 % rows])
        n1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= budget_s:
            break
    ncpu = os.cpu_count() or 1
    workers = max(1, min(ncpu, 16))
    with mp.get_context("spawn").Pool(workers) as pool:
        pool.map(_oracle_row, args[:workers], chunksize=1)      # start-up outside the timed region
        t0 = time.perf_counter()
        nn = 0
        while True:
            pool.map(_oracle_row, args, chunksize=1)
            nn += rows
            eln = time.perf_counter() - t0
            if eln >= budget_s:
                break
    model = _cpu_model()
    return {"value": nn / eln, "unit": "rows/s", "cores": workers, "kind": "oracle",
            "sample": f"{nn} decode rows (V={VOCAB}, k~U{{1..1024}}, top-p, Gumbel) in {eln:.1f} s over a "
                      f"pool of {workers} worker processes; os.cpu_count() = {ncpu}; CPU {model}",
            "single_core": {"value": n1 / el1, "unit": "rows/s", "cores": 1,
                            "sample": f"{n1} decode rows in {el1:.1f} s, one process"},
            "os_cpu_count": ncpu, "cpu_model": model}


# The other workloads: (generator, op, input buffers rotated so that each call reads cold
# data from HBM: R * bytes >= 512 MB where it fits, the MALL being 256 MB).
OTHER_CONFIGS = {
    "tiny": ("tiny", "sample", 4),
    "decode_topp_only": ("decode_topp_only", "sample", 16),
    "decode_logp": ("decode", "sample_logp", 16),
    "heavy": ("heavy", "sample", 16),
    "tie_stress": ("tie_stress", "sample", 8),
    "indexer_rows": ("indexer_rows", "topk", 32),
    "indexer_long": ("indexer_long", "topk", 128),
    "indexer_near_uniform": ("indexer_near_uniform", "topk", 900),
    "decode_topp_only_nok": ("decode_topp_only", "sample_nok", 16),
    "decode_rejection": ("decode", "rejection", 16),
    "decode_topp_only_rejection": ("decode_topp_only", "rejection", 16),
}


def other_config(name, args):
    """Time one non-headline workload: one JSON line of per-call kernel time and rates."""
    import numpy as np
    import torch

    import top_select_gumbel_amd as ts
    from top_select_gumbel_amd import workloads as wl

    gen, op, rot = OTHER_CONFIGS[name]
    dev = torch.device("cuda:0")
    lib = ts.load_library()
    b = getattr(wl, gen)()
    rows, vocab = b.logits.shape
    base = torch.from_numpy(b.logits).to(dev)
    bufs = [base] + [torch.roll(base, shifts=37 * i, dims=1).contiguous() for i in range(1, rot)]
    st = torch.empty(rows, dtype=torch.int32, device=dev)
    k = torch.from_numpy(b.k).to(dev)
    if op == "rejection":
        p = torch.from_numpy(b.p).to(dev)
        t = torch.from_numpy(b.t).to(dev)
        s = torch.from_numpy(b.seeds.view(np.int64)).to(dev)
        tok = torch.empty(rows, dtype=torch.int32, device=dev)
        rnd = torch.empty(rows, dtype=torch.int32, device=dev)
        call = lambda x, h: lib.ts_sample_rows_rejection(x, rows, vocab, vocab, k.data_ptr(), p.data_ptr(),
                                                         t.data_ptr(), None, s.data_ptr(), 32, tok.data_ptr(),
                                                         rnd.data_ptr(), st.data_ptr(), h)
        cname = "ts_sample_rows_rejection"
    elif op in ("sample", "sample_logp", "sample_nok"):
        p = torch.from_numpy(b.p).to(dev)
        t = torch.from_numpy(b.t).to(dev)
        seeds = b.seeds if b.seeds is not None else wl.heavy_launch_seeds(0, rows)
        s = torch.from_numpy(seeds.view(np.int64)).to(dev)
        tok = torch.empty(rows, dtype=torch.int32, device=dev)
        nb = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, rows, vocab, 0)
        ws = ts.workspace(nb, dev)
        fixed = (k.data_ptr(), p.data_ptr(), t.data_ptr(), s.data_ptr(), tok.data_ptr(), st.data_ptr(),
                 ws.data_ptr(), ws.numel())
        call = lambda x, h: lib.ts_sample_rows(x, rows, vocab, vocab, *fixed, h)
        cname = "ts_sample_rows"
        if op == "sample_nok":   # no top-k array: top-k off for every row (the nucleus pass)
            call = lambda x, h: lib.ts_sample_rows(x, rows, vocab, vocab, None, *fixed[1:], h)
            cname = "ts_sample_rows (top_k NULL)"
        if op == "sample_logp":
            lp = torch.empty(rows, dtype=torch.float32, device=dev)
            ls = torch.empty(rows, dtype=torch.float32, device=dev)
            call = lambda x, h: lib.ts_sample_rows_logp(x, rows, vocab, vocab, k.data_ptr(), p.data_ptr(),
                                                        t.data_ptr(), s.data_ptr(), tok.data_ptr(), lp.data_ptr(),
                                                        ls.data_ptr(), st.data_ptr(), ws.data_ptr(), ws.numel(), h)
            cname = "ts_sample_rows_logp"
    else:
        out = torch.empty((rows, b.k_max), dtype=torch.int32, device=dev)
        nb = lib.ts_workspace_bytes(ts.TS_OP_TOPK_SELECT, rows, vocab, b.k_max)
        ws = ts.workspace(nb, dev)
        call = lambda x, h: lib.ts_topk_select(x, rows, vocab, vocab, k.data_ptr(), b.k_max, out.data_ptr(),
                                               st.data_ptr(), ws.data_ptr(), ws.numel(), h)
        cname = "ts_topk_select"
    ptrs = [x.data_ptr() for x in bufs]
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream

    def timed(n, warm):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record(stream)
            rc = call(ptrs[0] if warm else ptrs[i % rot], h)
            ev[i][1].record(stream)
            if rc:
                raise RuntimeError(ts.ts_last_error())
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(e) for a, e in ev]) * 1e3   # us

    for i in range(args.warmup):
        call(ptrs[i % rot], h)
    torch.cuda.synchronize()
    us = timed(args.steps, False)
    warm_us = timed(min(args.steps, 200), True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(ptrs[i % rot], h)
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) / args.steps * 1e6
    assert int(st.abs().sum()) == 0, "rows reported errors"
    nbytes = rows * vocab * 4
    med = float(np.median(us))
    extra = {}
    if op == "rejection":
        r = rnd.cpu().numpy()
        extra = {"rounds_mean": float(r[r > 0].mean()) if (r > 0).any() else 0.0,
                 "rounds_max": int(r.max()), "fallback_rows": int((r < 0).sum())}
    print(json.dumps({
        "config": name, "op": cname, "rows": rows, "vocab": vocab, "input_buffers": rot,
        "bytes_per_call": nbytes, "steps": args.steps, "warmup": args.warmup,
        "kernel_us": {"median": med, "p10": float(np.percentile(us, 10)), "p90": float(np.percentile(us, 90))},
        "warm_kernel_us_median": float(np.median(warm_us)),
        "back_to_back_us_per_call": wall_us,
        "rows_per_s": rows / (wall_us * 1e-6),
        "effective_GBps_median": nbytes / (med * 1e-6) / 1e9,
        "frac_of_8TBps": nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "source_hash": source_hash(),
        **extra,
    }), flush=True)


def rejection_matrix(args):
    """The sampling matrix of mlxcel issue #901 ("Performance validation"): vocab {32000,
    65536, 151936} x batch {1, 4, 8} x filter {top-k 40, top-p 0.9, min-p 0.05, top-k 40 +
    top-p 0.9}, T = 1, the exact sampler (ts_sample_rows_minp) against the rejection sampler
    (ts_sample_rows_rejection). Inputs rotate over 512 MB so every call reads HBM. One JSON
    line per cell (median kernel time per call)."""
    import numpy as np
    import torch

    import top_select_gumbel_amd as ts
    from top_select_gumbel_amd import workloads as wl

    dev = torch.device("cuda:0")
    lib = ts.load_library()
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    filters = {"top-k 40": (40, 1.0, 0.0), "top-p 0.9": (None, 0.9, 0.0), "min-p 0.05": (None, 1.0, 0.05),
               "top-k 40 + top-p 0.9": (40, 0.9, 0.0)}

    def timed(call, ptrs, n):
        for i in range(20):
            call(ptrs[i % len(ptrs)])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record(stream)
            rc = call(ptrs[i % len(ptrs)])
            ev[i][1].record(stream)
            if rc:
                raise RuntimeError(ts.ts_last_error())
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(e) for a, e in ev])) * 1e3

    for vocab in (32000, 65536, 151936):
        for rows in (1, 4, 8):
            b = wl.decode(seed=2, rows=rows, vocab=vocab)
            rot = max(1, (512 << 20) // (rows * vocab * 4))
            big = torch.from_numpy(np.tile(b.logits.ravel(), rot)).to(dev)
            ptrs = [big.data_ptr() + i * rows * vocab * 4 for i in range(rot)]
            s = torch.from_numpy(b.seeds.view(np.int64)).to(dev)
            t = torch.ones(rows, dtype=torch.float32, device=dev)
            tok = torch.empty(rows, dtype=torch.int32, device=dev)
            rnd = torch.empty(rows, dtype=torch.int32, device=dev)
            st = torch.empty(rows, dtype=torch.int32, device=dev)
            nb = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, rows, vocab, 0)
            ws = ts.workspace(nb, dev)
            for fname, (kk, pp, mm) in filters.items():
                k = torch.full((rows,), kk if kk else vocab, dtype=torch.int32, device=dev)
                p = torch.full((rows,), pp, dtype=torch.float32, device=dev)
                mp = torch.full((rows,), mm, dtype=torch.float32, device=dev)
                # no top-k array when the filter has no top-k (the exact sampler's nucleus passes)
                kp = k.data_ptr() if kk else None
                exact = lambda x: lib.ts_sample_rows_minp(x, rows, vocab, vocab, kp, p.data_ptr(),
                                                          t.data_ptr(), mp.data_ptr(), s.data_ptr(), tok.data_ptr(),
                                                          st.data_ptr(), ws.data_ptr(), ws.numel(), h)
                rej = lambda x: lib.ts_sample_rows_rejection(x, rows, vocab, vocab, kp, p.data_ptr(),
                                                             t.data_ptr(), mp.data_ptr(), s.data_ptr(), 32,
                                                             tok.data_ptr(), rnd.data_ptr(), st.data_ptr(), h)
                us_exact = timed(exact, ptrs, args.steps)
                us_rej = timed(rej, ptrs, args.steps)
                r = rnd.cpu().numpy()
                assert int(st.abs().sum()) == 0, "rows reported errors"
                print(json.dumps({"config": "rejection_matrix", "vocab": vocab, "rows": rows, "filter": fname,
                                  "exact_us_median": us_exact, "rejection_us_median": us_rej,
                                  "rejection_over_exact": us_rej / us_exact,
                                  "rounds_last_call": r.tolist()}), flush=True)
            del big


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm-only", action="store_true")
    ap.add_argument("--config", default="decode", choices=["decode", "rejection_matrix"] + sorted(OTHER_CONFIGS),
                    help="decode (the headline line) or one of the other workloads, timed alone")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "rows are independent, so N GPUs would each take B/N rows of the same kernel.",
              file=sys.stderr)
        sys.exit(2)

    if args.config == "rejection_matrix":
        rejection_matrix(args)
        return
    if args.config != "decode":
        other_config(args.config, args)
        return

    import numpy as np
    import torch

    import top_select_gumbel_amd as ts
    from top_select_gumbel_amd import workloads as wl

    dev = torch.device("cuda:0")
    ts.load_library()
    batch = wl.decode()
    k = torch.from_numpy(batch.k).to(dev)
    p = torch.from_numpy(batch.p).to(dev)
    t = torch.from_numpy(batch.t).to(dev)
    s = torch.from_numpy(batch.seeds.view(np.int64)).to(dev)
    base = torch.from_numpy(batch.logits).to(dev)
    # distinct buffers: the same rows cyclically shifted per buffer (identical work per step)
    bufs = [base] + [torch.roll(base, shifts=37 * i, dims=1).contiguous() for i in range(1, ROTATE)]
    tok = torch.empty(ROWS, dtype=torch.int32, device=dev)
    st = torch.empty(ROWS, dtype=torch.int32, device=dev)
    lib = ts.load_library()
    nb = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, ROWS, VOCAB, 0)
    ws = ts.workspace(nb, dev)
    torch.cuda.synchronize()
    ptrs = [b.data_ptr() for b in bufs]
    fixed = (k.data_ptr(), p.data_ptr(), t.data_ptr(), s.data_ptr(), tok.data_ptr(), st.data_ptr(),
             ws.data_ptr(), ws.numel())

    def step(i, warm=False, stream_handle=None):
        # the C entry point itself, with pointers prepared once (no per-call tensor checks)
        h = torch.cuda.current_stream().cuda_stream if stream_handle is None else stream_handle
        rc = lib.ts_sample_rows(ptrs[0] if warm else ptrs[i % ROTATE], ROWS, VOCAB, VOCAB, *fixed, h)
        if rc:
            raise RuntimeError(ts.ts_last_error())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Per-launch kernel time with HIP events on the stream the kernel runs on.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = np.array([a.elapsed_time(b) for a, b in ev])

    # Whole-job throughput: K back-to-back steps, synchronised on both sides. One HIP event
    # pair on the same stream brackets the K calls: their average duration without the
    # per-call event records above (which add their own time to every call).
    torch.cuda.synchronize()
    e_bb0, e_bb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_bb0.record(stream)
    for i in range(args.steps):
        step(i)
    e_bb1.record(stream)
    torch.cuda.synchronize()
    wall_bb = time.perf_counter() - t0
    region_ms = e_bb0.elapsed_time(e_bb1) / args.steps

    # The same K steps captured once in a HIP graph and replayed (no host launch overhead).
    graph_ms_per_step = None
    try:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                h = torch.cuda.current_stream().cuda_stream
                for i in range(args.steps):
                    step(i, stream_handle=h)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        graph_ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    except Exception as exc:  # graph capture is an extra figure, not the headline
        print(f"bench.py: graph capture skipped: {exc}", file=sys.stderr)

    # Warm: the same buffer every step.
    warm = []
    for i in range(min(args.steps, 200)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(i, warm=True)
        b.record(stream)
        warm.append((a, b))
    torch.cuda.synchronize()
    warm_ms = np.array([a.elapsed_time(b) for a, b in warm])

    # A plain device copy of one logits buffer: the known-size kernel that calibrates the
    # FETCH_SIZE / WRITE_SIZE counters, and a read+write bandwidth reference.
    cp = torch.empty_like(base)
    cps = []
    for i in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        cp.copy_(bufs[i % ROTATE])
        b.record(stream)
        cps.append((a, b))
    torch.cuda.synchronize()
    copy_ms = float(np.median([a.elapsed_time(b) for a, b in cps]))

    # Known-size plain kernels for the FETCH_SIZE / WRITE_SIZE counters (profiles/): the
    # read-ceiling kernel below reads B*V*4 bytes and writes a few KB; the workspace fill
    # writes B*V*4 bytes. Both spread over every XCD, as the sampling kernels do. (The copy
    # above is one blit kernel whose counted share differs from run to run.)
    fill = torch.empty(BYTES_PER_CALL // 4, dtype=torch.int32, device=dev)
    for i in range(5):
        rc = lib.ts_workspace_init(fill.data_ptr(), BYTES_PER_CALL, stream.cuda_stream)
        if rc:
            raise RuntimeError(ts.ts_last_error())
    del fill

    # A plain read of the same buffers with the stream kernel's launch shape (the library's
    # diagnostic read kernel): the streaming ceiling the sampling call is compared against.
    # K back-to-back reads between one event pair, like region_us_per_call.
    acc = torch.empty(ts.read_ceiling_partials(ROWS * VOCAB), dtype=torch.float32, device=dev)
    for i in range(20):
        ts.ts_read_ceiling(bufs[i % ROTATE], acc)
    torch.cuda.synchronize()
    e_r0, e_r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_r0.record(stream)
    for i in range(args.steps):
        rc = lib.ts_read_ceiling(ptrs[i % ROTATE], ROWS * VOCAB, acc.data_ptr(), stream.cuda_stream)
        if rc:
            raise RuntimeError(ts.ts_last_error())
    e_r1.record(stream)
    torch.cuda.synchronize()
    read_ms = e_r0.elapsed_time(e_r1) / args.steps

    # A plain read of the same buffers (torch.sum) as a practical streaming ceiling.
    rd = []
    for i in range(min(args.steps, 100)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        bufs[i % ROTATE].sum()
        b.record(stream)
        rd.append((a, b))
    torch.cuda.synchronize()
    rd_ms = np.median([a.elapsed_time(b) for a, b in rd])

    assert int(st.abs().sum()) == 0, "rows reported errors"
    med = float(np.median(kern_ms))
    avg = float(kern_ms.mean())
    ms_per_step = wall_bb / args.steps * 1e3
    achieved = BYTES_PER_CALL / (region_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles()
    out = {
        "metric": "sampled rows/sec and effective HBM GB/s (% of peak) at V=151936, B=64",
        "value": ROWS * args.steps / wall_bb,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode sampling: B=64 x V=151936 fp32 logits 2.5*N(0,1) + 20 head "
                               "tokens (+8); k~U{1..1024}, p~U[0.5,1), T~U[0.5,1.5); Philox seeds per row",
                   "rows": ROWS, "vocab": VOCAB, "input_buffers": ROTATE, "op": "ts_sample_rows"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "region_us_per_call": region_ms * 1e3,
        # HBM passes over the logits per call (measured traffic / algorithmic bytes), from the
        # committed PMC summary while it matches the kernel sources
        "passes_per_row": None if traffic is None else traffic / BYTES_PER_CALL,
        "kernel_us": {"avg": avg * 1e3, "median": med * 1e3, "p10": float(np.percentile(kern_ms, 10)) * 1e3,
                      "p90": float(np.percentile(kern_ms, 90)) * 1e3},
        "warm_kernel_us_median": float(np.median(warm_ms)) * 1e3,
        "graph_us_per_step": None if graph_ms_per_step is None else graph_ms_per_step * 1e3,
        "effective_GBps_median": BYTES_PER_CALL / (med * 1e-3) / 1e9,
        "read_ceiling_GBps": BYTES_PER_CALL / (read_ms * 1e-3) / 1e9,
        "frac_of_read_ceiling": read_ms / region_ms,
        "torch_sum_read_GBps": BYTES_PER_CALL / (rd_ms * 1e-3) / 1e9,
        "copy_read_write_GBps": 2 * BYTES_PER_CALL / (copy_ms * 1e-3) / 1e9,
        "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(batch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
