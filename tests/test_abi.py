"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/mla8.h and include/mla8_aux.h declare, and refuses bad arguments on
the host before any HIP call; the Python binding refuses host tensors, wrong
dtypes and shapes before any address reaches the library.  No call here passes
validation, so no kernel is ever launched (the fake device pointers below are
never dereferenced)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from fp8_mla_latent_amd import mla8 as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("mla8.h", "mla8_aux.h")]

FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced
FAKE_MISALIGNED = ctypes.c_void_p(0x10004)


def declared_symbols():
    text = "".join(open(h).read() for h in HEADERS)
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
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert m.mla8_status_string(st) and m.mla8_status_string(st) != "unknown status"
    assert m.mla8_status_string(-99) == "unknown status"
    assert "gfx950" in m.mla8_version()


def dec(**kw):
    a = dict(codes=FAKE, scales=FAKE, t=100, lc=512, rc=64, ql=FAKE, qr=FAKE, h=64, sm=0.1,
             out=FAKE, lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return m.lib.mla8_decode(a["codes"], a["scales"], a["t"], a["lc"], a["rc"], a["ql"], a["qr"],
                             a["h"], a["sm"], a["out"], a["lse"], a["ws"], a["wsb"], None,
                             a.get("opts"))


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
    # a forced split count changes the plan and the size, for that call only
    o = m.Mla8Opts(2, None, None)
    need2 = m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 100, 64, 1, 512, ctypes.byref(o))
    assert need2 > need
    assert dec(wsb=need2 - 1, opts=ctypes.byref(o)) == m.MLA8_E_WORKSPACE
    assert dec(wsb=need - 1) == m.MLA8_E_WORKSPACE


def test_decode_sel_refuses():
    f = m.lib.mla8_decode_sel
    base = [FAKE, FAKE, 100, 512, 64, FAKE, 10, FAKE, FAKE, 64, 0.1, FAKE, None, FAKE, 1 << 30,
            None, None]
    for idx, val, want in [(5, None, m.MLA8_E_INVAL), (6, 0, m.MLA8_E_INVAL),
                           (6, -3, m.MLA8_E_INVAL), (5, ctypes.c_void_p(0x10002), m.MLA8_E_INVAL),
                           (14, 10, m.MLA8_E_WORKSPACE), (3, 100, m.MLA8_E_UNSUPPORTED)]:
        args = list(base)
        args[idx] = val
        assert f(*args) == want, (idx, val)


def test_batch_refuses():
    f = m.lib.mla8_batch
    base = [FAKE, FAKE, 100, 512, 64, FAKE, FAKE, 4, 96, 64, 0.1, FAKE, None, FAKE, 1 << 30, None,
            None]
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
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 256, 4) == 2     # chunks of at least 128 rows
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 4096, 128) == 32
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE_SEL, 2048, 64) == 32
    assert m.mla8_plan_splits(m.MLA8_OP_BATCH, 32768, 64, 64) == 2
    assert m.mla8_workspace_bytes(m.MLA8_OP_DECODE, 0, 64, 1, 512) == 0
    assert m.mla8_workspace_bytes(7, 10, 64, 1, 512) == 0
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 4096, 128, n_splits=5) == 5
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 100, 4, n_splits=5) == 2  # 64-row tiles
    assert m.mla8_plan_splits(m.MLA8_OP_DECODE, 4096, 128) == 32


def test_options_are_per_call():
    """The library keeps no state between calls: two interleaved callers with
    different split options (as two streams would be) each get their own plan
    and workspace size, and a caller with events armed changes nothing for a
    caller without."""
    o7 = m.Mla8Opts(7, None, None)
    o3 = m.Mla8Opts(3, None, None)
    armed = m.Mla8Opts(0, ctypes.c_void_p(0x1234), ctypes.c_void_p(0x5678))  # never recorded
    auto = m.lib.mla8_plan_splits(m.MLA8_OP_DECODE, 262144, 64, 1, None)
    ws_auto = m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 262144, 64, 1, 512, None)
    for _ in range(3):
        assert m.lib.mla8_plan_splits(m.MLA8_OP_DECODE, 262144, 64, 1, ctypes.byref(o7)) == 7
        assert m.lib.mla8_plan_splits(m.MLA8_OP_DECODE, 262144, 64, 1, ctypes.byref(o3)) == 3
        assert m.lib.mla8_plan_splits(m.MLA8_OP_DECODE, 262144, 64, 1, ctypes.byref(armed)) == auto
        assert m.lib.mla8_plan_splits(m.MLA8_OP_DECODE, 262144, 64, 1, None) == auto
        w7 = m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 262144, 64, 1, 512, ctypes.byref(o7))
        assert w7 == 2 * 7 * 64 * 4 + 7 * 64 * 512 * 4 + 3 * 0  # sections 256-byte rounded
        assert m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 262144, 64, 1, 512, None) == ws_auto
    # a refused call with options armed leaves the next default call unchanged
    assert dec(wsb=10, opts=ctypes.byref(armed)) == m.MLA8_E_WORKSPACE
    assert m.lib.mla8_plan_splits(m.MLA8_OP_DECODE, 262144, 64, 1, None) == auto


def test_append_decode_refuses():
    f = m.lib.mla8_append_decode
    t = ctypes.c_int64(10)
    base = [FAKE, FAKE, 100, ctypes.byref(t), FAKE, 1, 512, 64, FAKE, FAKE, 64, 0.1, FAKE, None,
            FAKE, 1 << 30, None, None]
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


def test_append_decode_noalloc_refuses():
    """Host checks only (no HIP call is reached): the usual refusals, and a
    call whose partials would not fit the static scratch."""
    f = m.lib.mla8_append_decode_noalloc
    t0 = 262143
    t = ctypes.c_int64(t0)
    base = [FAKE, FAKE, 300000, ctypes.byref(t), FAKE, 1, 512, 64, FAKE, FAKE, 64, 0.1, FAKE,
            None, None, None]
    too_many = m.Mla8Opts(1000, None, None)   # 1000 chunks x 64 heads x 514 x 4 B > 20 MiB
    ok_splits = m.Mla8Opts(128, None, None)
    assert m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 262144, 64, 1, 512,
                                      ctypes.byref(too_many)) > m.MLA8_SCRATCH_BYTES
    assert m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 262144, 64, 1, 512,
                                      ctypes.byref(ok_splits)) <= m.MLA8_SCRATCH_BYTES
    # the automatic plan fits for any head count up to 8192 (lc 512)
    for h in (1, 16, 64, 100, 128, 1000, 8192):
        assert m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 1 << 20, h, 1, 512, None) <= \
            m.MLA8_SCRATCH_BYTES, h
    for idx, val, want in [(4, None, m.MLA8_E_INVAL),         # no fresh rows
                           (5, 0, m.MLA8_E_INVAL),            # n_new = 0
                           (5, 65, m.MLA8_E_RANGE),           # more than the fused maximum
                           (2, t0, m.MLA8_E_CAPACITY),        # shadow full
                           (6, 500, m.MLA8_E_UNSUPPORTED),
                           (12, None, m.MLA8_E_INVAL),        # no out
                           (15, ctypes.byref(too_many), m.MLA8_E_SCRATCH)]:
        args = list(base)
        args[idx] = val
        assert f(*args) == want, (idx, val)
        assert t.value == t0  # never advanced on an error
    assert "scratch" in m.mla8_status_string(m.MLA8_E_SCRATCH)


def test_index_topk_refuses():
    f = m.lib.mla8_index_topk
    ws = m.lib.mla8_workspace_bytes(m.MLA8_OP_INDEX, 1000, 64, 1, 128, None)
    assert ws >= 1000 * 12 + 4096 * 4
    base = [FAKE, FAKE, 1000, 128, FAKE, FAKE, 64, 100, FAKE, None, FAKE, ws, None, None]
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
    ws = m.lib.mla8_workspace_bytes(m.MLA8_OP_DECODE, 100, 64, 1, 448, None)
    base = [FAKE, FAKE, 100, 448, 64, FAKE, FAKE, 64, 0.1, FAKE, None, FAKE, ws, None, None]
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
            FAKE, 1 << 30, None, None]
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
    ws = m.lib.mla8_workspace_bytes(m.MLA8_OP_BATCH, 100, 16, 4, 448, None)
    base = [FAKE, FAKE, 100, 448, 64, FAKE, FAKE, 4, 96, 16, 0.1, FAKE, None, FAKE, ws, None, None]
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


def test_test_encode_pk_refuses():
    f = m.lib.mla8_test_encode_pk
    assert f(None, 8, FAKE, None) == m.MLA8_E_INVAL
    assert f(FAKE, 8, None, None) == m.MLA8_E_INVAL
    assert f(FAKE, 6, FAKE, None) == m.MLA8_E_INVAL        # not a multiple of 4
    assert f(FAKE, -4, FAKE, None) == m.MLA8_E_INVAL
    assert f(FAKE_MISALIGNED, 8, FAKE, None) == m.MLA8_E_INVAL
    assert f(FAKE, 0, FAKE, None) == m.MLA8_OK             # nothing to do, nothing launched


# ---------------------------------------------------------------------------
# The binding's own checks: a host tensor, a wrong dtype or shape, or a row
# count beyond the buffer is refused in Python, before the C ABI sees an address.

import torch  # noqa: E402


def _cpu(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("call", [
    lambda: m.mla8_quantize_rows(_cpu((4, 576), torch.float32), 512, 64),
    lambda: m.mla8_append(_cpu((8, 576), torch.uint8), _cpu((8,), torch.float32), 0,
                          _cpu((1, 576), torch.float32), 512, 64),
    lambda: m.mla8_decode(_cpu((8, 576), torch.uint8), _cpu((8,), torch.float32), 8, 512, 64,
                          _cpu((4, 512), torch.float32), _cpu((4, 64), torch.float32), 0.1),
    lambda: m.mla8_append_decode(_cpu((8, 576), torch.uint8), _cpu((8,), torch.float32), 7,
                                 _cpu((1, 576), torch.float32), 512, 64,
                                 _cpu((4, 512), torch.float32), _cpu((4, 64), torch.float32), 0.1),
    lambda: m.mla8_decode_sel(_cpu((8, 576), torch.uint8), _cpu((8,), torch.float32), 8, 512, 64,
                              _cpu((3,), torch.int32), _cpu((4, 512), torch.float32),
                              _cpu((4, 64), torch.float32), 0.1),
    lambda: m.mla8_batch(_cpu((8, 576), torch.uint8), _cpu((8,), torch.float32), 8, 512, 64,
                         _cpu((2, 4, 512), torch.float32), _cpu((2, 4, 64), torch.float32), 6,
                         0.1),
    lambda: m.mla8_index_topk(_cpu((8, 128), torch.uint8), _cpu((8,), torch.float32),
                              _cpu((16, 128), torch.float32), _cpu((16,), torch.float32), 4),
    lambda: m.mla8_test_encode(_cpu((8,), torch.float32)),
    lambda: m.mla8_test_encode_pk(_cpu((8,), torch.float32)),
    lambda: m.mla8_stream_read(_cpu((64,), torch.uint8), _cpu((32768,), torch.int32)),
])
def test_binding_refuses_host_tensors(call):
    with pytest.raises(ValueError, match="device"):
        call()


class _FakeDev:
    """Stands in for a device tensor in the checks that come after the device
    test (dtype, shape, rows): only the attributes the checks read."""

    def __init__(self, shape, dtype):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.is_cuda = True
        self.device = torch.device("cuda", 0)

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return True


def test_binding_checks_dtype_shape_and_rows(monkeypatch):
    monkeypatch.setattr(m, "_TENSOR", _FakeDev)
    codes, scales = _FakeDev((8, 576), torch.uint8), _FakeDev((8,), torch.float32)
    ql, qr = _FakeDev((4, 512), torch.float32), _FakeDev((4, 64), torch.float32)
    with pytest.raises(ValueError, match="torch.float32"):   # f64 query
        m.mla8_decode(codes, scales, 8, 512, 64, _FakeDev((4, 512), torch.float64), qr, 0.1)
    with pytest.raises(ValueError, match="shape"):           # row width of another shape
        m.mla8_decode(_FakeDev((8, 512), torch.uint8), scales, 8, 512, 64, ql, qr, 0.1)
    with pytest.raises(ValueError, match="shape"):           # q_rope of another width
        m.mla8_decode(codes, scales, 8, 512, 64, ql, _FakeDev((4, 32), torch.float32), 0.1)
    with pytest.raises(ValueError, match="t_rows"):          # more rows than the buffer
        m.mla8_decode(codes, scales, 9, 512, 64, ql, qr, 0.1)
    with pytest.raises(ValueError, match="shape"):           # scales of another length
        m.mla8_decode(codes, _FakeDev((7,), torch.float32), 8, 512, 64, ql, qr, 0.1)
    with pytest.raises(ValueError, match="torch.int32"):     # int64 selection
        m.mla8_decode_sel(codes, scales, 8, 512, 64, _FakeDev((3,), torch.int64), ql, qr, 0.1)
    with pytest.raises(ValueError, match="t_rows"):          # batch rows beyond the buffer
        m.mla8_batch(codes, scales, 9, 512, 64, _FakeDev((2, 4, 512), torch.float32),
                     _FakeDev((2, 4, 64), torch.float32), 7, 0.1)
