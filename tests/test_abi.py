"""Host-side checks of the C ABI that need no GPU: the library loads, exports every symbol
include/*.h declares, sizes workspaces, and rejects bad arguments before touching a
device (no compute calls are made here)."""
import ctypes
import glob
import os
import re
import threading

import pytest

import top_select_gumbel_amd as ts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(ts_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ts.LIB_PATH):
        pytest.fail("libtopselect.so is not built (python -m top_select_gumbel_amd.build)")
    return ts.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(ts.EXPORTED) == names


def test_workspace_sizes(lib):
    a = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, 64, 151936, 0)
    b = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, 128, 151936, 0)
    assert a > 0 and b > a and a % 256 == 0
    assert lib.ts_workspace_bytes(ts.TS_OP_TOPK_SELECT, 1, 1 << 20, 2048) > 0
    assert lib.ts_workspace_bytes(7, 1, 10, 1) == 0            # unknown op
    assert lib.ts_workspace_bytes(0, 1, 0, 1) == 0             # vocab < 1
    assert lib.ts_workspace_bytes(0, -1, 10, 1) == 0           # rows < 0
    assert lib.ts_workspace_bytes(0, 1, (1 << 30) + 1, 1) == 0  # vocab too large


def test_bad_arguments_fail_before_any_device_work(lib):
    c = ctypes
    nullp = None
    fake = c.c_void_p(0x1000)                      # never dereferenced on these paths
    rc = lib.ts_topk_select(nullp, 1, 10, 10, fake, 4, fake, None, fake, 1 << 20, None)
    assert rc == ts.TS_ERR_INVALID_ARG and "NULL" in lib.ts_last_error().decode()
    rc = lib.ts_topk_select(fake, 1, 10, 5, fake, 4, fake, None, fake, 1 << 20, None)
    assert rc == ts.TS_ERR_INVALID_ARG and "stride" in lib.ts_last_error().decode()
    rc = lib.ts_topk_select(fake, 1, 10, 10, fake, 0, fake, None, fake, 1 << 20, None)
    assert rc == ts.TS_ERR_INVALID_ARG
    rc = lib.ts_topk_select(fake, 1, 10, 10, None, 4, fake, None, fake, 1 << 20, None)
    assert rc == ts.TS_ERR_INVALID_ARG
    rc = lib.ts_sample_rows(fake, 2, 10, 10, None, None, None, None, fake, None, fake, 1 << 20, None)
    assert rc == ts.TS_ERR_INVALID_ARG                    # seed required
    rc = lib.ts_topp_mask(fake, 2, 10, 10, None, None, None, None, None, None, fake, 1 << 20, None)
    assert rc == ts.TS_ERR_INVALID_ARG                    # out_kept required
    rc = lib.ts_topp_mask(fake, 2, 0, 10, None, None, None, fake, None, None, fake, 1 << 20, None)
    assert rc == ts.TS_ERR_INVALID_ARG                    # vocab < 1
    # workspace checks come before any device query
    rc = lib.ts_sample_rows(fake, 2, 10, 10, None, None, None, fake, fake, None, None, 1 << 20, None)
    assert rc == ts.TS_ERR_WORKSPACE
    rc = lib.ts_sample_rows(fake, 2, 10, 10, None, None, None, fake, fake, None, c.c_void_p(0x1001), 1 << 20, None)
    assert rc == ts.TS_ERR_WORKSPACE and "aligned" in lib.ts_last_error().decode()
    rc = lib.ts_sample_rows(fake, 2, 10, 10, None, None, None, fake, fake, None, fake, 16, None)
    assert rc == ts.TS_ERR_WORKSPACE and "needs" in lib.ts_last_error().decode()
    # zero rows is a no-op that succeeds, with any pointers (an empty tensor's are NULL)
    assert lib.ts_sample_rows(fake, 0, 10, 10, None, None, None, None, None, None, None, 0, None) == ts.TS_OK
    assert lib.ts_sample_rows(None, 0, 10, 10, None, None, None, None, None, None, None, 0, None) == ts.TS_OK
    assert lib.ts_topk_select(None, 0, 10, 10, None, 4, None, None, None, 0, None) == ts.TS_OK
    assert lib.ts_topp_mask(None, 0, 10, 10, None, None, None, None, None, None, None, 0, None) == ts.TS_OK
    assert lib.ts_sample_rows_rejection(None, 0, 10, 10, None, None, None, None, None, 8, None, None, None,
                                        None) == ts.TS_OK
    # ... but not with an invalid shape
    assert lib.ts_sample_rows(None, 0, 0, 10, None, None, None, None, None, None, None, 0, None) == ts.TS_ERR_INVALID_ARG


def test_status_strings_and_knobs(lib):
    for code in (0, -1, -2, -3, -4, 1, 2, 3, 4):
        assert lib.ts_status_string(code).decode() != "unknown status"
    assert lib.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 12345) == -1      # not a multiple of 64
    old = lib.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 2048)
    assert old == 0
    small = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, 4, 100000, 0)
    assert lib.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 0) == 2048
    big = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, 4, 100000, 0)
    assert small != big
    assert lib.ts_debug_set(ts.TS_KNOB_NUCLEUS_PASSES, 1) == 0
    assert lib.ts_debug_set(ts.TS_KNOB_NUCLEUS_PASSES, 0) == 1
    assert lib.ts_debug_set(99, 1) == -1


def test_knobs_belong_to_the_calling_thread(lib):
    # a chunk size forced on another thread changes neither this thread's setting nor the
    # workspace size it computes
    base = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, 4, 100000, 0)
    seen = {}

    def other():
        seen["old"] = lib.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 1024)
        seen["ws"] = lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, 4, 100000, 0)
        seen["main_during"] = None

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["old"] == 0 and seen["ws"] != base
    assert lib.ts_workspace_bytes(ts.TS_OP_SAMPLE_ROWS, 4, 100000, 0) == base
    assert lib.ts_debug_set(ts.TS_KNOB_CHUNK_ELEMS, 0) == 0          # this thread never changed


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ts.TopSelectError):
        ts.load_library(str(tmp_path / "missing.so"))
