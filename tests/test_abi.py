"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/mla8.h declares, and refuses bad arguments on the host before any HIP
call.  No call here passes validation, so no kernel is ever launched (the fake
device pointers below are never dereferenced)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from fp8_mla_latent_amd import mla8 as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla8.h")

FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced
FAKE_MISALIGNED = ctypes.c_void_p(0x10004)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MLA8_API\s+[\w\s\*]+?\b(mla8_\w+)\s*\(", text)))


def test_header_declares_the_product_calls():
    syms = declared_symbols()
    for name in ("mla8_quantize_rows", "mla8_append", "mla8_decode", "mla8_append_decode",
                 "mla8_decode_sel", "mla8_batch", "mla8_index_topk", "mla8_quantize_rows_mx",
                 "mla8_append_mx", "mla8_decode_mx", "mla8_decode_sel_mx", "mla8_workspace_bytes",
                 "mla8_status_string"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(m._LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(m.EXPORTED)


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert m.mla8_status_string(st) and m.mla8_status_string(st) != "unknown status"
    assert m.mla8_status_string(-99) == "unknown status"
    assert "gfx950" in m.mla8_version()


def dec(**kw):
    a = dict(codes=FAKE, scales=FAKE, t=100, lc=512, rc=64, ql=FAKE, qr=FAKE, h=64, sm=0.1,
             out=FAKE, lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return m.lib.mla8_decode(a["codes"], a["scales"], a["t"], a["lc"], a["rc"], a["ql"], a["qr"],
                             a["h"], a["sm"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(codes=None), m.MLA8_E_INVAL),
    (dict(scales=None), m.MLA8_E_INVAL),
    (dict(ql=None), m.MLA8_E_INVAL),
    (dict(qr=None), m.MLA8_E_INVAL),
    (dict(out=None), m.MLA8_E_INVAL),
    (dict(t=0), m.MLA8_E_INVAL),
    (dict(t=-5), m.MLA8_E_INVAL),
    (dict(t=1 << 31), m.MLA8_E_INVAL),
    (dict(h=0), m.MLA8_E_INVAL),
    (dict(sm=float("nan")), m.MLA8_E_INVAL),
    (dict(sm=float("inf")), m.MLA8_E_INVAL),
    (dict(codes=FAKE_MISALIGNED), m.MLA8_E_INVAL),
    (dict(lc=500), m.MLA8_E_UNSUPPORTED),
    (dict(lc=1024), m.MLA8_E_UNSUPPORTED),
    (dict(lc=0), m.MLA8_E_UNSUPPORTED),
    (dict(rc=8), m.MLA8_E_UNSUPPORTED),
    (dict(rc=144), m.MLA8_E_UNSUPPORTED),
    (dict(lc=512, rc=144), m.MLA8_E_UNSUPPORTED),
    (dict(ws=None), m.MLA8_E_WORKSPACE),
    (dict(wsb=100), m.MLA8_E_WORKSPACE),
])
def test_decode_refuses(kw, want):
    assert dec(**kw) == want


def test_decode_workspace_exact_boundary():
    need = m.mla8_workspace_bytes(m.MLA8_OP_DECODE, 100, 64, 1, 512)
    assert need > 0
    assert dec(wsb=need - 1) == m.MLA8_E_WORKSPACE


def test_decode_sel_refuses():
    f = m.lib.mla8_decode_sel
    base = [FAKE, FAKE, 100, 512, 64, FAKE, 10, FAKE, FAKE, 64, 0.1, FAKE, None, FAKE, 1 << 30,
            None]
    for idx, val, want in [(5, None, m.MLA8_E_INVAL), (6, 0, m.MLA8_E_INVAL),
                           (6, -3, m.MLA8_E_INVAL), (5, ctypes.c_void_p(0x10002), m.MLA8_E_INVAL),
                           (14, 10, m.MLA8_E_WORKSPACE), (3, 100, m.MLA8_E_UNSUPPORTED)]:
        args = list(base)
        args[idx] = val
        assert f(*args) == want, (idx, val)


def test_batch_refuses():
    f = m.lib.mla8_batch
    base = [FAKE, FAKE, 100, 512, 64, FAKE, FAKE, 4, 96, 64, 0.1, FAKE, None, FAKE, 1 << 30, None]
    for idx, val, want in [(7, 0, m.MLA8_E_INVAL), (8, -1, m.MLA8_E_INVAL),
                           (8, 97, m.MLA8_E_RANGE), (2, 50, m.MLA8_E_RANGE),
                           (14, 64, m.MLA8_E_WORKSPACE), (0, None, m.MLA8_E_INVAL)]:
        args = list(base)
        args[idx] = val
        assert f(*args) == want, (idx, val)


def test_quantize_and_append_refuse():
    q = m.lib.mla8_quantize_rows
    assert q(None, 4, 512, 64, FAKE, FAKE, None) == m.MLA8_E_INVAL
    assert q(FAKE, -1, 512, 64, FAKE, FAKE, None) == m.MLA8_E_INVAL
    assert q(FAKE, 4, 500, 64, FAKE, FAKE, None) == m.MLA8_E_UNSUPPORTED
    assert q(FAKE_MISALIGNED, 4, 512, 64, FAKE, FAKE, None) == m.MLA8_E_INVAL
    assert q(FAKE, 0, 512, 64, FAKE, FAKE, None) == m.MLA8_OK
    a = m.lib.mla8_append
    t = ctypes.c_int64(10)
    assert a(FAKE, FAKE, 12, ctypes.byref(t), FAKE, 3, 512, 64, None) == m.MLA8_E_CAPACITY
    assert t.value == 10
    assert a(FAKE, FAKE, 12, None, FAKE, 1, 512, 64, None) == m.MLA8_E_INVAL
    t2 = ctypes.c_int64(13)
    assert a(FAKE, FAKE, 12, ctypes.byref(t2), FAKE, 0, 512, 64, None) == m.MLA8_E_INVAL
    t3 = ctypes.c_int64(12)
    assert a(FAKE, FAKE, 12, ctypes.byref(t3), FAKE, 0, 512, 64, None) == m.MLA8_OK
    assert t3.value == 12


def test_plans_and_workspace_sizes():
    # long-context decode: 128 chunks of 2048 rows x 2 head groups = 256 workgroups
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 262144, 64) == 128
    assert m.mla8_workspace_bytes(m.MLA8_OP_DECODE, 262144, 64, 1, 512) == \
        2 * 128 * 64 * 4 + 128 * 64 * 512 * 4
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 256, 4) == 1
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 4096, 128) == 16
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE_SEL, 2048, 64) == 32
    assert m.mla8_plan_splits(m.MLA8_OP_BATCH, 32768, 64, 64) == 2
    assert m.mla8_workspace_bytes(m.MLA8_OP_DECODE, 0, 64, 1, 512) == 0
    assert m.mla8_workspace_bytes(7, 10, 64, 1, 512) == 0
    prev = m.mla8_force_splits(5)
    try:
        assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 4096, 128) == 5
        assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 100, 4) == 2  # clamped to the 64-row tiles
    finally:
        m.mla8_force_splits(prev)
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 4096, 128) == 16


def test_append_decode_refuses():
    f = m.lib.mla8_append_decode
    t = ctypes.c_int64(10)
    base = [FAKE, FAKE, 100, ctypes.byref(t), FAKE, 1, 512, 64, FAKE, FAKE, 64, 0.1, FAKE, None,
            FAKE, 1 << 30, None]
    for idx, val, want in [(4, None, m.MLA8_E_INVAL),         # no fresh rows
                           (5, 0, m.MLA8_E_INVAL),            # n_new = 0
                           (5, 65, m.MLA8_E_RANGE),           # more than the fused maximum
                           (2, 10, m.MLA8_E_CAPACITY),        # shadow full
                           (4, FAKE_MISALIGNED, m.MLA8_E_INVAL),
                           (6, 500, m.MLA8_E_UNSUPPORTED),
                           (8, None, m.MLA8_E_INVAL),         # no q_lat
                           (15, 10, m.MLA8_E_WORKSPACE)]:
        args = list(base)
        args[idx] = val
        assert f(*args) == want, (idx, val)
        assert t.value == 10  # never advanced on an error


def test_index_topk_refuses():
    f = m.lib.mla8_index_topk
    ws = m.lib.mla8_workspace_bytes(m.MLA8_OP_INDEX, 1000, 64, 1, 128)
    assert ws >= 1000 * 12 + 4096 * 4
    base = [FAKE, FAKE, 1000, 128, FAKE, FAKE, 64, 100, FAKE, None, FAKE, ws, None]
    for idx, val, want in [(0, None, m.MLA8_E_INVAL),        # no keys
                           (4, None, m.MLA8_E_INVAL),        # no query
                           (5, None, m.MLA8_E_INVAL),        # no weights
                           (8, None, m.MLA8_E_INVAL),        # no output
                           (2, 0, m.MLA8_E_INVAL),           # no rows
                           (7, 0, m.MLA8_E_INVAL),           # top_k = 0
                           (3, 64, m.MLA8_E_UNSUPPORTED),    # ihd other than 128
                           (6, 40, m.MLA8_E_UNSUPPORTED),    # n_ih not a multiple of 16
                           (6, 80, m.MLA8_E_UNSUPPORTED),    # more than 64 heads
                           (7, 4097, m.MLA8_E_UNSUPPORTED),  # top_k beyond the LDS sort
                           (2, (1 << 24) + 1, m.MLA8_E_UNSUPPORTED),  # more rows than 2^24
                           (4, FAKE_MISALIGNED, m.MLA8_E_INVAL),
                           (11, ws - 1, m.MLA8_E_WORKSPACE),
                           (10, None, m.MLA8_E_WORKSPACE)]:
        args = list(base)
        args[idx] = val
        assert f(*args) == want, (idx, val)


def test_mixed_refuses():
    q = m.lib.mla8_quantize_rows_mx
    assert q(FAKE, 4, 512, 64, FAKE, FAKE, None) == m.MLA8_E_UNSUPPORTED
    assert q(FAKE, 4, 448, 32, FAKE, FAKE, None) == m.MLA8_E_UNSUPPORTED
    assert q(None, 4, 448, 64, FAKE, FAKE, None) == m.MLA8_E_INVAL
    assert q(FAKE, -1, 448, 64, FAKE, FAKE, None) == m.MLA8_E_INVAL
    assert q(FAKE_MISALIGNED, 4, 448, 64, FAKE, FAKE, None) == m.MLA8_E_INVAL
    t = ctypes.c_int64(3)
    a = m.lib.mla8_append_mx
    assert a(FAKE, FAKE, 4, ctypes.byref(t), FAKE, 2, 448, 64, None) == m.MLA8_E_CAPACITY
    assert a(FAKE, FAKE, 4, ctypes.byref(t), FAKE, 1, 448, 48, None) == m.MLA8_E_UNSUPPORTED
    assert t.value == 3
    d = m.lib.mla8_decode_mx
    ws = m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 100, 64, 1, 448)
    base = [FAKE, FAKE, 100, 448, 64, FAKE, FAKE, 64, 0.1, FAKE, None, FAKE, ws, None]
    for idx, val, want in [(3, 512, m.MLA8_E_UNSUPPORTED), (0, None, m.MLA8_E_INVAL),
                           (2, 0, m.MLA8_E_INVAL), (12, ws - 1, m.MLA8_E_WORKSPACE),
                           (6, None, m.MLA8_E_INVAL)]:
        args = list(base)
        args[idx] = val
        assert d(*args) == want, (idx, val)


def test_mixed_step_and_batch_refuse():
    f = m.lib.mla8_append_decode_mx
    t = ctypes.c_int64(10)
    base = [FAKE, FAKE, 100, ctypes.byref(t), FAKE, 1, 448, 64, FAKE, FAKE, 64, 0.1, FAKE, None,
            FAKE, 1 << 30, None]
    for idx, val, want in [(6, 512, m.MLA8_E_UNSUPPORTED),   # the e4m3 shape is not mixed
                           (7, 32, m.MLA8_E_UNSUPPORTED),
                           (4, None, m.MLA8_E_INVAL),         # no fresh rows
                           (5, 65, m.MLA8_E_RANGE),           # more than the fused maximum
                           (2, 10, m.MLA8_E_CAPACITY),        # shadow full
                           (4, FAKE_MISALIGNED, m.MLA8_E_INVAL),
                           (15, 10, m.MLA8_E_WORKSPACE)]:
        args = list(base)
        args[idx] = val
        assert f(*args) == want, (idx, val)
        assert t.value == 10
    b = m.lib.mla8_batch_mx
    ws = m.lib.mla8_workspace_bytes(m.MLA8_OP_BATCH, 100, 16, 4, 448)
    base = [FAKE, FAKE, 100, 448, 64, FAKE, FAKE, 4, 96, 16, 0.1, FAKE, None, FAKE, ws, None]
    for idx, val, want in [(3, 512, m.MLA8_E_UNSUPPORTED), (7, 0, m.MLA8_E_INVAL),
                           (8, 97, m.MLA8_E_RANGE), (14, ws - 1, m.MLA8_E_WORKSPACE),
                           (5, None, m.MLA8_E_INVAL)]:
        args = list(base)
        args[idx] = val
        assert b(*args) == want, (idx, val)


def test_stream_read_refuses():
    f = m.lib.mla8_stream_read
    assert f(None, 64, FAKE, None) == m.MLA8_E_INVAL
    assert f(FAKE, 64, None, None) == m.MLA8_E_INVAL
    assert f(FAKE_MISALIGNED, 64, FAKE, None) == m.MLA8_E_INVAL
    assert f(FAKE, 40, FAKE, None) == m.MLA8_E_INVAL      # not a multiple of 16
    assert f(FAKE, -16, FAKE, None) == m.MLA8_E_INVAL
    assert f(FAKE, 64, FAKE_MISALIGNED, None) == m.MLA8_E_INVAL
