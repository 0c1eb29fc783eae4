"""Python binding of the gfx950 batched top-k / top-p / Gumbel-max sampler (libtopselect.so).

Argument marshalling only: every step of the sampling path runs in the HIP library. The
functions take torch tensors that already live on the GPU and enqueue on the current torch
stream. There is no CPU fallback: if the library is missing, calls raise.

Names mirror the C ABI in include/topselect.h (ts_debug_set: the test hooks of
include/topselect_testing.h).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtopselect.so")

TS_OK = 0
TS_ERR_INVALID_ARG = -1
TS_ERR_WORKSPACE = -2
TS_ERR_UNSUPPORTED = -3
TS_ERR_LAUNCH = -4
TS_ROW_OK = 0
TS_ROW_NONFINITE = 1
TS_ROW_BAD_K = 2
TS_ROW_BAD_P = 3
TS_ROW_BAD_T = 4
TS_ROW_BAD_MINP = 5
TS_ORDER_INDEX = 0
TS_ORDER_VALUE = 1
TS_OP_TOPK_SELECT = 0
TS_OP_TOPP_MASK = 1
TS_OP_SAMPLE_ROWS = 2
TS_KNOB_CHUNK_ELEMS = 1
TS_KNOB_FORCE_EXACT = 2
TS_KNOB_DIRECT = 3
TS_KNOB_NUCLEUS_PASSES = 4

EXPORTED = (
    "ts_workspace_bytes", "ts_workspace_init", "ts_topk_select", "ts_topk_select_rows", "ts_topp_mask",
    "ts_sample_rows", "ts_sample_rows_noalloc", "ts_sample_rows_logp", "ts_topp_mask_minp", "ts_sample_rows_minp", "ts_sample_rows_rejection", "ts_gumbel_noise", "ts_noise_transform", "ts_read_ceiling", "ts_debug_set", "ts_status_string", "ts_last_error",
)

_lib = None
_lib_lock = threading.Lock()


class TopSelectError(RuntimeError):
    pass


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libtopselect.so (built in-tree by top_select_gumbel_amd.build) and declare its ABI."""
    global _lib
    with _lib_lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise TopSelectError(
                f"{p} is missing: build it with `python -m top_select_gumbel_amd.build` "
                "(there is no CPU fallback)")
        lib = ctypes.CDLL(p)
        c = ctypes
        vp, i64, i32, sz = c.c_void_p, c.c_int64, c.c_int32, c.c_size_t
        lib.ts_workspace_bytes.argtypes = [c.c_int, i64, i64, i32]
        lib.ts_workspace_bytes.restype = sz
        lib.ts_workspace_init.argtypes = [vp, sz, vp]
        lib.ts_workspace_init.restype = c.c_int
        lib.ts_topk_select.argtypes = [vp, i64, i64, i64, vp, i32, vp, vp, vp, sz, vp]
        lib.ts_topk_select.restype = c.c_int
        lib.ts_topk_select_rows.argtypes = [vp, i64, i64, i64, vp, vp, i32, c.c_int, vp, vp, vp, vp, sz, vp]
        lib.ts_topk_select_rows.restype = c.c_int
        lib.ts_topp_mask.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ts_topp_mask.restype = c.c_int
        lib.ts_sample_rows.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ts_sample_rows.restype = c.c_int
        lib.ts_sample_rows_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.ts_sample_rows_noalloc.restype = c.c_int
        lib.ts_sample_rows_logp.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ts_sample_rows_logp.restype = c.c_int
        lib.ts_topp_mask_minp.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ts_topp_mask_minp.restype = c.c_int
        lib.ts_sample_rows_minp.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ts_sample_rows_minp.restype = c.c_int
        lib.ts_sample_rows_rejection.restype = c.c_int
        lib.ts_sample_rows_rejection.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
        lib.ts_gumbel_noise.argtypes = [c.c_uint64, i32, vp, i64, vp, vp, vp, vp]
        lib.ts_noise_transform.restype = c.c_int
        lib.ts_noise_transform.argtypes = [vp, i64, vp, vp, vp]
        lib.ts_gumbel_noise.restype = c.c_int
        lib.ts_read_ceiling.argtypes = [vp, i64, vp, vp]
        lib.ts_read_ceiling.restype = c.c_int
        lib.ts_debug_set.argtypes = [c.c_int, i64]
        lib.ts_debug_set.restype = i64
        lib.ts_status_string.argtypes = [c.c_int]
        lib.ts_status_string.restype = c.c_char_p
        lib.ts_last_error.argtypes = []
        lib.ts_last_error.restype = c.c_char_p
        if path is None:
            _lib = lib
        return lib


def _check(rc: int) -> None:
    if rc != TS_OK:
        lib = load_library()
        raise TopSelectError(f"{lib.ts_status_string(rc).decode()} ({rc}): {lib.ts_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


# Workspaces are cached per (device, stream); a call reuses the cached buffer when it is
# large enough. The kernels leave the counter region zeroed after every call.
_ws_cache = {}


def workspace(nbytes: int, device):
    import torch
    key = (str(device), _stream())
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def ts_workspace_bytes(op: int, rows: int, vocab: int, k_max: int = 0) -> int:
    return int(load_library().ts_workspace_bytes(op, rows, vocab, k_max))


def _rows_view(x):
    if x.dim() != 2:
        raise TopSelectError("logits must be a 2-D tensor with unit column stride")
    if not x.is_cuda or x.dtype.is_complex or str(x.dtype) != "torch.float32":
        raise TopSelectError("logits must be a float32 CUDA/HIP tensor")
    if x.shape[0] == 0:   # an empty batch: strides carry no layout (numpy gives them as 0)
        return 0, x.shape[1], x.shape[1]
    if x.stride(1) != 1:
        raise TopSelectError("logits must be a 2-D tensor with unit column stride")
    return x.shape[0], x.shape[1], x.stride(0)


def _opt(t, dtype_name: str, rows: int):
    if t is None:
        return None
    if str(t.dtype) != dtype_name or not t.is_cuda or t.numel() != rows or not t.is_contiguous():
        raise TopSelectError(f"per-row parameter must be a contiguous {dtype_name} device tensor of {rows}")
    return t


def ts_topk_select(keys, k, k_max: int, row_len: Optional[int] = None):
    """Top-k select: returns (out_idx int32 [rows, k_max] ascending ids / -1 pads, status int32)."""
    import torch
    lib = load_library()
    rows, cols, stride = _rows_view(keys)
    v = cols if row_len is None else int(row_len)
    k = _opt(k, "torch.int32", rows)
    out = torch.empty((rows, k_max), dtype=torch.int32, device=keys.device)
    st = torch.empty(rows, dtype=torch.int32, device=keys.device)
    nb = lib.ts_workspace_bytes(TS_OP_TOPK_SELECT, rows, v, k_max)
    ws = workspace(nb, keys.device)
    _check(lib.ts_topk_select(_ptr(keys), rows, v, stride, _ptr(k), k_max, _ptr(out), _ptr(st),
                              _ptr(ws), ws.numel(), _stream()))
    return out, st


def ts_topk_select_rows(keys, k, k_max: int, lengths=None, order: int = 0, offsets=None,
                        row_len: Optional[int] = None):
    """Top-k over each row's valid prefix (lengths), ids ascending (order 0) or value-ordered
    (order 1), shifted by offsets: returns (out_idx int32 [rows, k_max], status int32)."""
    import torch
    lib = load_library()
    rows, cols, stride = _rows_view(keys)
    v = cols if row_len is None else int(row_len)
    k = _opt(k, "torch.int32", rows)
    lengths = _opt(lengths, "torch.int32", rows)
    offsets = _opt(offsets, "torch.int32", rows)
    out = torch.empty((rows, k_max), dtype=torch.int32, device=keys.device)
    st = torch.empty(rows, dtype=torch.int32, device=keys.device)
    nb = lib.ts_workspace_bytes(TS_OP_TOPK_SELECT, rows, v, k_max)
    ws = workspace(nb, keys.device)
    _check(lib.ts_topk_select_rows(_ptr(keys), rows, v, stride, _ptr(lengths), _ptr(k), k_max, int(order),
                                   _ptr(offsets), _ptr(out), _ptr(st), _ptr(ws), ws.numel(), _stream()))
    return out, st


def ts_topp_mask(logits, top_k=None, top_p=None, temperature=None, want_mask: bool = True):
    """Top-k then top-p: returns (kept int32 [rows], mask uint8 [rows, vocab] or None, status)."""
    import torch
    lib = load_library()
    rows, v, stride = _rows_view(logits)
    top_k = _opt(top_k, "torch.int32", rows)
    top_p = _opt(top_p, "torch.float32", rows)
    temperature = _opt(temperature, "torch.float32", rows)
    kept = torch.empty(rows, dtype=torch.int32, device=logits.device)
    mask = torch.empty((rows, v), dtype=torch.uint8, device=logits.device) if want_mask else None
    st = torch.empty(rows, dtype=torch.int32, device=logits.device)
    nb = lib.ts_workspace_bytes(TS_OP_TOPP_MASK, rows, v, 0)
    ws = workspace(nb, logits.device)
    _check(lib.ts_topp_mask(_ptr(logits), rows, v, stride, _ptr(top_k), _ptr(top_p),
                            _ptr(temperature), _ptr(kept), _ptr(mask), _ptr(st), _ptr(ws),
                            ws.numel(), _stream()))
    return kept, mask, st


def ts_sample_rows(logits, top_k, top_p, temperature, seed, out_token=None, status=None):
    """Sample one token per row: returns (tokens int32 [rows], status int32 [rows])."""
    import torch
    lib = load_library()
    rows, v, stride = _rows_view(logits)
    top_k = _opt(top_k, "torch.int32", rows)
    top_p = _opt(top_p, "torch.float32", rows)
    temperature = _opt(temperature, "torch.float32", rows)
    if seed is None or str(seed.dtype) not in ("torch.uint64", "torch.int64") or seed.numel() != rows:
        raise TopSelectError("seed must be a uint64/int64 device tensor with one entry per row")
    tok = out_token if out_token is not None else torch.empty(rows, dtype=torch.int32, device=logits.device)
    st = status if status is not None else torch.empty(rows, dtype=torch.int32, device=logits.device)
    nb = lib.ts_workspace_bytes(TS_OP_SAMPLE_ROWS, rows, v, 0)
    ws = workspace(nb, logits.device)
    _check(lib.ts_sample_rows(_ptr(logits), rows, v, stride, _ptr(top_k), _ptr(top_p),
                              _ptr(temperature), _ptr(seed), _ptr(tok), _ptr(st), _ptr(ws),
                              ws.numel(), _stream()))
    return tok, st


def ts_sample_rows_noalloc(logits, top_k, top_p, temperature, seed, out_token=None, status=None):
    """ts_sample_rows without a workspace (the library's static scratch): same results.
    Allocates only the output tensors when they are not given."""
    import torch
    lib = load_library()
    rows, v, stride = _rows_view(logits)
    top_k = _opt(top_k, "torch.int32", rows)
    top_p = _opt(top_p, "torch.float32", rows)
    temperature = _opt(temperature, "torch.float32", rows)
    if seed is None or str(seed.dtype) not in ("torch.uint64", "torch.int64") or seed.numel() != rows:
        raise TopSelectError("seed must be a uint64/int64 device tensor with one entry per row")
    tok = out_token if out_token is not None else torch.empty(rows, dtype=torch.int32, device=logits.device)
    st = status if status is not None else torch.empty(rows, dtype=torch.int32, device=logits.device)
    _check(lib.ts_sample_rows_noalloc(_ptr(logits), rows, v, stride, _ptr(top_k), _ptr(top_p),
                                      _ptr(temperature), _ptr(seed), _ptr(tok), _ptr(st), _stream()))
    return tok, st


def ts_sample_rows_logp(logits, top_k, top_p, temperature, seed, want_lse: bool = True):
    """Sample one token per row with its logprob: returns (tokens int32, logp fp32,
    lse fp32 or None, status int32), each [rows]."""
    import torch
    lib = load_library()
    rows, v, stride = _rows_view(logits)
    top_k = _opt(top_k, "torch.int32", rows)
    top_p = _opt(top_p, "torch.float32", rows)
    temperature = _opt(temperature, "torch.float32", rows)
    if seed is None or str(seed.dtype) not in ("torch.uint64", "torch.int64") or seed.numel() != rows:
        raise TopSelectError("seed must be a uint64/int64 device tensor with one entry per row")
    tok = torch.empty(rows, dtype=torch.int32, device=logits.device)
    logp = torch.empty(rows, dtype=torch.float32, device=logits.device)
    lse = torch.empty(rows, dtype=torch.float32, device=logits.device) if want_lse else None
    st = torch.empty(rows, dtype=torch.int32, device=logits.device)
    nb = lib.ts_workspace_bytes(TS_OP_SAMPLE_ROWS, rows, v, 0)
    ws = workspace(nb, logits.device)
    _check(lib.ts_sample_rows_logp(_ptr(logits), rows, v, stride, _ptr(top_k), _ptr(top_p),
                                   _ptr(temperature), _ptr(seed), _ptr(tok), _ptr(logp), _ptr(lse),
                                   _ptr(st), _ptr(ws), ws.numel(), _stream()))
    return tok, logp, lse, st


def ts_topp_mask_minp(logits, top_k, top_p, temperature, min_p, want_mask: bool = True):
    """Top-k, top-p then min-p: returns (kept int32 [rows], mask uint8 [rows, vocab] or None, status)."""
    import torch
    lib = load_library()
    rows, v, stride = _rows_view(logits)
    top_k = _opt(top_k, "torch.int32", rows)
    top_p = _opt(top_p, "torch.float32", rows)
    temperature = _opt(temperature, "torch.float32", rows)
    min_p = _opt(min_p, "torch.float32", rows)
    if min_p is None:
        raise TopSelectError("min_p is required")
    kept = torch.empty(rows, dtype=torch.int32, device=logits.device)
    mask = torch.empty((rows, v), dtype=torch.uint8, device=logits.device) if want_mask else None
    st = torch.empty(rows, dtype=torch.int32, device=logits.device)
    nb = lib.ts_workspace_bytes(TS_OP_TOPP_MASK, rows, v, 0)
    ws = workspace(nb, logits.device)
    _check(lib.ts_topp_mask_minp(_ptr(logits), rows, v, stride, _ptr(top_k), _ptr(top_p),
                                 _ptr(temperature), _ptr(min_p), _ptr(kept), _ptr(mask), _ptr(st),
                                 _ptr(ws), ws.numel(), _stream()))
    return kept, mask, st


def ts_sample_rows_minp(logits, top_k, top_p, temperature, min_p, seed):
    """Sample after top-k, top-p and min-p: returns (tokens int32 [rows], status int32 [rows])."""
    import torch
    lib = load_library()
    rows, v, stride = _rows_view(logits)
    top_k = _opt(top_k, "torch.int32", rows)
    top_p = _opt(top_p, "torch.float32", rows)
    temperature = _opt(temperature, "torch.float32", rows)
    min_p = _opt(min_p, "torch.float32", rows)
    if min_p is None:
        raise TopSelectError("min_p is required")
    if seed is None or str(seed.dtype) not in ("torch.uint64", "torch.int64") or seed.numel() != rows:
        raise TopSelectError("seed must be a uint64/int64 device tensor with one entry per row")
    tok = torch.empty(rows, dtype=torch.int32, device=logits.device)
    st = torch.empty(rows, dtype=torch.int32, device=logits.device)
    nb = lib.ts_workspace_bytes(TS_OP_SAMPLE_ROWS, rows, v, 0)
    ws = workspace(nb, logits.device)
    _check(lib.ts_sample_rows_minp(_ptr(logits), rows, v, stride, _ptr(top_k), _ptr(top_p),
                                   _ptr(temperature), _ptr(min_p), _ptr(seed), _ptr(tok), _ptr(st),
                                   _ptr(ws), ws.numel(), _stream()))
    return tok, st


def ts_sample_rows_rejection(logits, top_k, top_p, temperature, min_p, seed, max_rounds: int = 32):
    """Dual-pivot rejection sampling: returns (tokens int32, rounds int32, status int32), each
    [rows]; rounds is the accepting round (1-based), 0 for greedy or rejected rows, -1 when the
    row reached max_rounds and took the exact fallback draw."""
    import torch
    lib = load_library()
    rows, v, stride = _rows_view(logits)
    top_k = _opt(top_k, "torch.int32", rows)
    top_p = _opt(top_p, "torch.float32", rows)
    temperature = _opt(temperature, "torch.float32", rows)
    min_p = _opt(min_p, "torch.float32", rows)
    if seed is None or str(seed.dtype) not in ("torch.uint64", "torch.int64") or seed.numel() != rows:
        raise TopSelectError("seed must be a uint64/int64 device tensor with one entry per row")
    tok = torch.empty(rows, dtype=torch.int32, device=logits.device)
    rnd = torch.empty(rows, dtype=torch.int32, device=logits.device)
    st = torch.empty(rows, dtype=torch.int32, device=logits.device)
    _check(lib.ts_sample_rows_rejection(_ptr(logits), rows, v, stride, _ptr(top_k), _ptr(top_p),
                                        _ptr(temperature), _ptr(min_p), _ptr(seed), int(max_rounds),
                                        _ptr(tok), _ptr(rnd), _ptr(st), _stream()))
    return tok, rnd, st


def ts_gumbel_noise(seed: int, row: int, tokens):
    """The sampler's (Philox word, u, g) for each token id of `row` under `seed`."""
    import torch
    lib = load_library()
    n = tokens.numel()
    word = torch.empty(n, dtype=torch.int32, device=tokens.device)
    u = torch.empty(n, dtype=torch.float32, device=tokens.device)
    g = torch.empty(n, dtype=torch.float32, device=tokens.device)
    _check(lib.ts_gumbel_noise(int(seed) & 0xFFFFFFFFFFFFFFFF, int(row), _ptr(tokens), n, _ptr(word),
                               _ptr(u), _ptr(g), _stream()))
    return word, u, g


def ts_noise_transform(words):
    """The sampler's (u, g) for given 32-bit words (an int32/uint32 device tensor)."""
    import torch
    lib = load_library()
    n = words.numel()
    u = torch.empty(n, dtype=torch.float32, device=words.device)
    g = torch.empty(n, dtype=torch.float32, device=words.device)
    _check(lib.ts_noise_transform(_ptr(words), n, _ptr(u), _ptr(g), _stream()))
    return u, g


def read_ceiling_partials(n: int) -> int:
    """Length of the partial-sum array ts_read_ceiling writes for n floats."""
    return 4 * ((n + 8191) // 8192)


def ts_read_ceiling(x, out=None):
    """Plain streaming read of a float32 device tensor (contiguous, 16-byte aligned) with the
    stream kernel's launch shape. Returns the per-wave fp32 partial sums (`out`, allocated when
    None: read_ceiling_partials(x.numel()) floats). A bandwidth reference."""
    import torch
    lib = load_library()
    if str(x.dtype) != "torch.float32" or not x.is_contiguous():
        raise TopSelectError("x must be a contiguous float32 tensor")
    if out is None:
        out = torch.empty(max(1, read_ceiling_partials(x.numel())), dtype=torch.float32, device=x.device)
    _check(lib.ts_read_ceiling(_ptr(x), x.numel(), _ptr(out), _stream()))
    return out


def ts_debug_set(knob: int, value: int) -> int:
    return int(load_library().ts_debug_set(knob, value))


def ts_status_string(status: int) -> str:
    return load_library().ts_status_string(status).decode()


def ts_last_error() -> str:
    return load_library().ts_last_error().decode()
