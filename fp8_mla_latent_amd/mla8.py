"""Thin Python binding over libmla8.so (include/mla8.h, include/mla8_aux.h),
same names as the C ABI.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels.  The
library must be built (``python -m fp8_mla_latent_amd.build``); importing this
module without it raises, there is no fallback path.

The C ABI takes raw device addresses and cannot tell a host pointer, a wrong
dtype or a too-small buffer from a good one, so every wrapper here checks its
tensors first (device, dtype, contiguity, shapes, and, where the call passes no
capacity, the row count against the buffer's rows) and raises ValueError before
any address reaches the library.  What the library can check itself (an
append beyond cap_rows, queries beyond t_rows) is left to its status codes.

Per-call options (the C struct mla8_opts): ``n_splits`` forces the number of
row chunks of the split-T plan (0 = automatic), ``events`` = (before, after)
torch.cuda.Event pair recorded around the split-T partial kernel (the
indexer's score kernel for mla8_index_topk), ``f32_scores`` scores of f32
grade also for the e4m3 512/64 decode, selected-row decode and causal batch,
which by default attend with the query's lo term quantized to e4m3 (see
mla8_opts in include/mla8.h).
Nothing is kept between calls.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla8.so")

MLA8_OK = 0
MLA8_E_INVAL = -1
MLA8_E_RANGE = -2
MLA8_E_CAPACITY = -3
MLA8_E_WORKSPACE = -4
MLA8_E_UNSUPPORTED = -5
MLA8_E_HIP = -6
MLA8_E_IO = -7
MLA8_E_SCRATCH = -8
MLA8_SCRATCH_BYTES = 20 << 20
MLA8_OP_DECODE = 0
MLA8_OP_DECODE_SEL = 1
MLA8_OP_BATCH = 2
MLA8_OP_INDEX = 3
MLA8_STREAM_WORDS = 32768

# Every symbol declared in include/mla8.h and include/mla8_aux.h.
EXPORTED = ("mla8_quantize_rows", "mla8_append", "mla8_decode", "mla8_append_decode",
            "mla8_decode_sel", "mla8_batch", "mla8_quantize_rows_mx", "mla8_append_mx",
            "mla8_decode_mx", "mla8_decode_sel_mx", "mla8_append_decode_mx", "mla8_batch_mx",
            "mla8_append_decode_noalloc", "mla8_index_topk", "mla8_kvfile_create",
            "mla8_kvfile_info", "mla8_kvfile_append", "mla8_kvfile_load",
            "mla8_workspace_bytes", "mla8_plan_splits",
            "mla8_status_string", "mla8_version", "mla8_test_encode", "mla8_test_encode_pk",
            "mla8_stream_read")


class Mla8Opts(ctypes.Structure):
    """struct mla8_opts (include/mla8.h)."""
    _fields_ = [("n_splits", ctypes.c_int32), ("ev_before", ctypes.c_void_p),
                ("ev_after", ctypes.c_void_p), ("f32_scores", ctypes.c_int32)]


class Mla8Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: status {status}: {mla8_status_string(status)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libmla8.so not built at {_LIB_PATH}; run "
                          "`python -m fp8_mla_latent_amd.build` (no fallback path exists)")
    L = ctypes.CDLL(_LIB_PATH)
    P, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                            ctypes.c_size_t)
    O = ctypes.POINTER(Mla8Opts)
    sig = {
        "mla8_quantize_rows": (ctypes.c_int, [P, i64, i32, i32, P, P, P]),
        "mla8_append": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64, i32, i32, P]),
        "mla8_decode": (ctypes.c_int, [P, P, i64, i32, i32, P, P, i32, f32, P, P, P, sz, P, O]),
        "mla8_append_decode": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64, i32, i32,
                                              P, P, i32, f32, P, P, P, sz, P, O]),
        "mla8_append_decode_noalloc": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64,
                                                      i32, i32, P, P, i32, f32, P, P, P, O]),
        "mla8_decode_sel": (ctypes.c_int,
                            [P, P, i64, i32, i32, P, i64, P, P, i32, f32, P, P, P, sz, P, O]),
        "mla8_batch": (ctypes.c_int,
                       [P, P, i64, i32, i32, P, P, i32, i64, i32, f32, P, P, P, sz, P, O]),
        "mla8_quantize_rows_mx": (ctypes.c_int, [P, i64, i32, i32, P, P, P]),
        "mla8_append_mx": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64, i32, i32, P]),
        "mla8_decode_mx": (ctypes.c_int,
                           [P, P, i64, i32, i32, P, P, i32, f32, P, P, P, sz, P, O]),
        "mla8_decode_sel_mx": (ctypes.c_int,
                               [P, P, i64, i32, i32, P, i64, P, P, i32, f32, P, P, P, sz, P, O]),
        "mla8_append_decode_mx": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64, i32,
                                                 i32, P, P, i32, f32, P, P, P, sz, P, O]),
        "mla8_batch_mx": (ctypes.c_int,
                          [P, P, i64, i32, i32, P, P, i32, i64, i32, f32, P, P, P, sz, P, O]),
        "mla8_index_topk": (ctypes.c_int,
                            [P, P, i64, i32, P, P, i32, i32, P, P, P, sz, P, O]),
        "mla8_kvfile_create": (ctypes.c_int, [ctypes.c_char_p, i32, i32, i32]),
        "mla8_kvfile_info": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(i32),
                                            ctypes.POINTER(i32), ctypes.POINTER(i32),
                                            ctypes.POINTER(i32), ctypes.POINTER(i64)]),
        "mla8_kvfile_append": (ctypes.c_int, [ctypes.c_char_p, i32, P, P, i64, i64, i32, i32,
                                              i32, P]),
        "mla8_kvfile_load": (ctypes.c_int, [ctypes.c_char_p, i32, P, P, i64,
                                            ctypes.POINTER(i64), i32, i32, i32, P, sz, P]),
        "mla8_workspace_bytes": (sz, [i32, i64, i32, i32, i32, O]),
        "mla8_plan_splits": (i32, [i32, i64, i32, i32, O]),
        "mla8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "mla8_version": (ctypes.c_char_p, []),
        "mla8_test_encode": (ctypes.c_int, [P, i64, P, P]),
        "mla8_test_encode_pk": (ctypes.c_int, [P, i64, P, P]),
        "mla8_stream_read": (ctypes.c_int, [P, i64, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


# ---------------------------------------------------------------------------
# argument checks (host side, before any address reaches the library)

_TENSOR = torch.Tensor  # the accepted tensor type (tests substitute a stand-in)


def _dev(t, name: str, dtype: torch.dtype, shape=None, device=None) -> torch.Tensor:
    """t must be a contiguous device tensor of `dtype`; `shape` entries of None
    match any size.  Returns t."""
    if not isinstance(t, _TENSOR):
        raise ValueError(f"mla8: {name} must be a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"mla8: {name} must be a device (cuda) tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"mla8: {name} is on {t.device}, the call's other tensors on {device}")
    if t.dtype != dtype:
        raise ValueError(f"mla8: {name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"mla8: {name} must be contiguous")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and s != d for s, d in zip(shape, t.shape)):
            want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
            raise ValueError(f"mla8: {name} has shape {list(t.shape)}, expected {want}")
    return t


def _shadow(codes, scales, row_bytes: int, device=None):
    """A shadow (codes [cap, row_bytes] uint8, scales [cap] f32); returns cap."""
    _dev(codes, "kv_codes", torch.uint8, (None, row_bytes), device)
    cap = codes.shape[0]
    _dev(scales, "kv_scales", torch.float32, (cap,), codes.device)
    return cap


def _queries(q_lat, q_rope, lead: tuple, lc: int, rc: int, device):
    _dev(q_lat, "q_lat", torch.float32, (*lead, lc), device)
    if rc > 0:
        _dev(q_rope, "q_rope", torch.float32, (*lead, rc), device)
    elif q_rope is not None:
        _dev(q_rope, "q_rope", torch.float32, (*lead, 0), device)


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("mla8: tensors must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int | None:
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status: int, call: str) -> None:
    if status != MLA8_OK:
        raise Mla8Error(status, call)


def _opts(n_splits: int = 0, events=None, f32_scores: bool = False):
    """A Mla8Opts for one call, or None for the defaults.  events: (before,
    after) torch.cuda.Event; torch creates an event's hipEvent on its first
    record(), so both must have been recorded once."""
    if not n_splits and events is None and not f32_scores:
        return None
    o = Mla8Opts(int(n_splits), None, None, 1 if f32_scores else 0)
    if events is not None:
        raw = []
        for ev in events:
            if ev is None:
                raw.append(None)
                continue
            if not ev.cuda_event:
                raise ValueError("mla8: record the event once before passing it")
            raw.append(ev.cuda_event)
        o.ev_before, o.ev_after = raw
    return ctypes.byref(o), o  # keep the struct alive with its reference


def _o(opts):
    return None if opts is None else opts[0]


def mla8_status_string(status: int) -> str:
    return lib.mla8_status_string(status).decode()


def mla8_version() -> str:
    return lib.mla8_version().decode()


def mla8_workspace_bytes(op: int, rows: int, n_heads: int, n_q: int, lc: int,
                         n_splits: int = 0) -> int:
    return int(lib.mla8_workspace_bytes(op, rows, n_heads, n_q, lc, _o(_opts(n_splits))))


def mla8_plan_splits(op: int, rows: int, n_heads: int, n_q: int = 1, n_splits: int = 0) -> int:
    return int(lib.mla8_plan_splits(op, rows, n_heads, n_q, _o(_opts(n_splits))))


def _workspace(op, rows, n_heads, n_q, lc, device, workspace, n_splits):
    need = mla8_workspace_bytes(op, rows, n_heads, n_q, lc, n_splits)
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _dev(workspace, "workspace", torch.uint8, (None,), device)
    return workspace


def _out_lse(out, lse, lead: tuple, lc: int, device, want_lse: bool):
    if out is None:
        out = torch.empty((*lead, lc), dtype=torch.float32, device=device)
    else:
        _dev(out, "out", torch.float32, (*lead, lc), device)
    if lse is None and want_lse:
        lse = torch.empty(lead, dtype=torch.float32, device=device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32, lead, device)
    return out, lse


# ---------------------------------------------------------------------------
# quantizer and shadow

def mla8_quantize_rows(x: torch.Tensor, lc: int, rc: int, codes: torch.Tensor | None = None,
                       scales: torch.Tensor | None = None):
    """f32 rows [n, lc+rc] -> (uint8 codes [n, lc+rc], f32 scales [n])."""
    _dev(x, "x", torch.float32, (None, lc + rc))
    n = x.shape[0]
    if codes is None:
        codes = torch.empty((n, lc + rc), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n,), dtype=torch.float32, device=x.device)
    _dev(codes, "codes", torch.uint8, (n, lc + rc), x.device)
    _dev(scales, "scales", torch.float32, (n,), x.device)
    _check(lib.mla8_quantize_rows(_ptr(x), n, lc, rc, _ptr(codes), _ptr(scales), _stream(x)),
           "mla8_quantize_rows")
    return codes, scales


def mla8_append(kv_codes: torch.Tensor, kv_scales: torch.Tensor, t_rows: int, x: torch.Tensor,
                lc: int, rc: int) -> int:
    """Quantize rows x into the shadow at [t_rows, t_rows + n); returns the new t_rows."""
    cap = _shadow(kv_codes, kv_scales, lc + rc)
    _dev(x, "x", torch.float32, (None, lc + rc), kv_codes.device)
    t = ctypes.c_int64(t_rows)
    _check(lib.mla8_append(_ptr(kv_codes), _ptr(kv_scales), cap, ctypes.byref(t),
                           _ptr(x), x.shape[0], lc, rc, _stream(x)), "mla8_append")
    return int(t.value)


def mla8_quantize_rows_mx(x: torch.Tensor, lc: int, rc: int, rows=None, scales=None):
    """Mixed rows: f32 [n, lc + rc] -> (uint8 rows [n, lc + 2 rc], f32 scales [n])."""
    _dev(x, "x", torch.float32, (None, lc + rc))
    n = x.shape[0]
    if rows is None:
        rows = torch.empty((n, lc + 2 * rc), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n,), dtype=torch.float32, device=x.device)
    _dev(rows, "rows", torch.uint8, (n, lc + 2 * rc), x.device)
    _dev(scales, "scales", torch.float32, (n,), x.device)
    _check(lib.mla8_quantize_rows_mx(_ptr(x), n, lc, rc, _ptr(rows), _ptr(scales), _stream(x)),
           "mla8_quantize_rows_mx")
    return rows, scales


def mla8_append_mx(kv_rows, kv_scales, t_rows: int, x, lc: int, rc: int) -> int:
    cap = _shadow(kv_rows, kv_scales, lc + 2 * rc)
    _dev(x, "x", torch.float32, (None, lc + rc), kv_rows.device)
    t = ctypes.c_int64(t_rows)
    _check(lib.mla8_append_mx(_ptr(kv_rows), _ptr(kv_scales), cap, ctypes.byref(t),
                              _ptr(x), x.shape[0], lc, rc, _stream(x)), "mla8_append_mx")
    return int(t.value)


# ---------------------------------------------------------------------------
# attention

def _decode_call(fn: str, row_bytes: int, kv, kv_scales, t_rows, lc, rc, q_lat, q_rope,
                 sm_scale, out, lse, workspace, want_lse, n_splits, events, f32_scores=False):
    cap = _shadow(kv, kv_scales, row_bytes)
    dev = kv.device
    if not (1 <= int(t_rows) <= cap):
        raise ValueError(f"mla8: t_rows = {t_rows} outside the shadow's [1, {cap}] rows")
    _dev(q_lat, "q_lat", torch.float32, (None, lc), dev)
    h = q_lat.shape[0]
    _queries(q_lat, q_rope, (h,), lc, rc, dev)
    out, lse = _out_lse(out, lse, (h,), lc, dev, want_lse)
    ws = _workspace(MLA8_OP_DECODE, t_rows, h, 1, lc, dev, workspace, n_splits)
    o = _opts(n_splits, events, f32_scores)
    _check(getattr(lib, fn)(_ptr(kv), _ptr(kv_scales), t_rows, lc, rc, _ptr(q_lat), _ptr(q_rope),
                            h, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                            _stream(q_lat), _o(o)), fn)
    return out, lse


def mla8_decode(kv_codes, kv_scales, t_rows: int, lc: int, rc: int, q_lat, q_rope,
                sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True,
                n_splits: int = 0, events=None, f32_scores: bool = False):
    """Dense decode over shadow rows [0, t_rows): returns (out [H, lc], lse [H] or None)."""
    return _decode_call("mla8_decode", lc + rc, kv_codes, kv_scales, t_rows, lc, rc, q_lat,
                        q_rope, sm_scale, out, lse, workspace, want_lse, n_splits, events,
                        f32_scores)


def mla8_decode_mx(kv_rows, kv_scales, t_rows: int, lc: int, rc: int, q_lat, q_rope,
                   sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True,
                   n_splits: int = 0, events=None, f32_scores: bool = False):
    """Dense decode over mixed rows [0, t_rows): (out [H, lc], lse [H] or None)."""
    return _decode_call("mla8_decode_mx", lc + 2 * rc, kv_rows, kv_scales, t_rows, lc, rc,
                        q_lat, q_rope, sm_scale, out, lse, workspace, want_lse, n_splits, events,
                        f32_scores)


def mla8_append_decode(kv_codes, kv_scales, t_rows: int, x_new, lc: int, rc: int, q_lat, q_rope,
                       sm_scale: float, out=None, lse=None, workspace=None,
                       want_lse: bool = True, n_splits: int = 0, events=None,
                       f32_scores: bool = False, _fn: str = "mla8_append_decode"):
    """Append x_new [n, lc+rc] at rows [t_rows, t_rows + n) and decode over all
    t_rows + n rows in one launch: returns (out, lse, new t_rows)."""
    mixed = _fn == "mla8_append_decode_mx"
    cap = _shadow(kv_codes, kv_scales, lc + (2 if mixed else 1) * rc)
    dev = kv_codes.device
    _dev(x_new, "x_new", torch.float32, (None, lc + rc), dev)
    n = x_new.shape[0]
    _dev(q_lat, "q_lat", torch.float32, (None, lc), dev)
    h = q_lat.shape[0]
    _queries(q_lat, q_rope, (h,), lc, rc, dev)
    out, lse = _out_lse(out, lse, (h,), lc, dev, want_lse)
    ws = _workspace(MLA8_OP_DECODE, t_rows + n, h, 1, lc, dev, workspace, n_splits)
    o = _opts(n_splits, events, f32_scores)
    t = ctypes.c_int64(t_rows)
    _check(getattr(lib, _fn)(_ptr(kv_codes), _ptr(kv_scales), cap, ctypes.byref(t), _ptr(x_new),
                             n, lc, rc, _ptr(q_lat), _ptr(q_rope), h, float(sm_scale),
                             _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(q_lat), _o(o)),
           _fn)
    return out, lse, int(t.value)


def mla8_append_decode_noalloc(kv_codes, kv_scales, t_rows: int, x_new, lc: int, rc: int,
                               q_lat, q_rope, sm_scale: float, out, lse=None,
                               n_splits: int = 0, f32_scores: bool = False) -> int:
    """As mla8_append_decode with the library's static scratch instead of a
    workspace; allocates nothing, so `out` ([H, lc] f32) must be given (lse
    [H] f32 optional).  Returns the new t_rows."""
    cap = _shadow(kv_codes, kv_scales, lc + rc)
    dev = kv_codes.device
    _dev(x_new, "x_new", torch.float32, (None, lc + rc), dev)
    _dev(q_lat, "q_lat", torch.float32, (None, lc), dev)
    h = q_lat.shape[0]
    _queries(q_lat, q_rope, (h,), lc, rc, dev)
    _dev(out, "out", torch.float32, (h, lc), dev)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (h,), dev)
    o = _opts(n_splits, None, f32_scores)
    t = ctypes.c_int64(t_rows)
    _check(lib.mla8_append_decode_noalloc(_ptr(kv_codes), _ptr(kv_scales), cap, ctypes.byref(t),
                                          _ptr(x_new), x_new.shape[0], lc, rc, _ptr(q_lat),
                                          _ptr(q_rope), h, float(sm_scale), _ptr(out),
                                          _ptr(lse), _stream(q_lat), _o(o)),
           "mla8_append_decode_noalloc")
    return int(t.value)


def mla8_append_decode_mx(kv_rows, kv_scales, t_rows: int, x_new, lc: int, rc: int, q_lat,
                          q_rope, sm_scale: float, out=None, lse=None, workspace=None,
                          want_lse: bool = True, n_splits: int = 0, events=None,
                          f32_scores: bool = False):
    """As mla8_append_decode over mixed rows (kv_rows [cap, lc + 2 rc])."""
    return mla8_append_decode(kv_rows, kv_scales, t_rows, x_new, lc, rc, q_lat, q_rope, sm_scale,
                              out, lse, workspace, want_lse, n_splits, events, f32_scores,
                              _fn="mla8_append_decode_mx")


def _sel_call(fn: str, row_bytes: int, kv, kv_scales, t_rows, lc, rc, sel, q_lat, q_rope,
              sm_scale, out, lse, workspace, want_lse, n_splits, events, f32_scores=False):
    cap = _shadow(kv, kv_scales, row_bytes)
    dev = kv.device
    if not (1 <= int(t_rows) <= cap):
        raise ValueError(f"mla8: t_rows = {t_rows} outside the shadow's [1, {cap}] rows")
    _dev(sel, "sel", torch.int32, (None,), dev)
    ns = sel.shape[0]
    _dev(q_lat, "q_lat", torch.float32, (None, lc), dev)
    h = q_lat.shape[0]
    _queries(q_lat, q_rope, (h,), lc, rc, dev)
    out, lse = _out_lse(out, lse, (h,), lc, dev, want_lse)
    ws = _workspace(MLA8_OP_DECODE_SEL, ns, h, 1, lc, dev, workspace, n_splits)
    o = _opts(n_splits, events, f32_scores)
    _check(getattr(lib, fn)(_ptr(kv), _ptr(kv_scales), t_rows, lc, rc, _ptr(sel), ns,
                            _ptr(q_lat), _ptr(q_rope), h, float(sm_scale), _ptr(out), _ptr(lse),
                            _ptr(ws), ws.numel(), _stream(q_lat), _o(o)), fn)
    return out, lse


def mla8_decode_sel(kv_codes, kv_scales, t_rows: int, lc: int, rc: int, sel, q_lat, q_rope,
                    sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True,
                    n_splits: int = 0, events=None, f32_scores: bool = False):
    """Decode over the selected absolute rows sel [ns] (int32; entries outside
    [0, t_rows) are skipped by the kernel)."""
    return _sel_call("mla8_decode_sel", lc + rc, kv_codes, kv_scales, t_rows, lc, rc, sel, q_lat,
                     q_rope, sm_scale, out, lse, workspace, want_lse, n_splits, events,
                     f32_scores)


def mla8_decode_sel_mx(kv_rows, kv_scales, t_rows: int, lc: int, rc: int, sel, q_lat, q_rope,
                       sm_scale: float, out=None, lse=None, workspace=None,
                       want_lse: bool = True, n_splits: int = 0, events=None,
                       f32_scores: bool = False):
    """Decode over the selected mixed rows sel (int32 device tensor)."""
    return _sel_call("mla8_decode_sel_mx", lc + 2 * rc, kv_rows, kv_scales, t_rows, lc, rc, sel,
                     q_lat, q_rope, sm_scale, out, lse, workspace, want_lse, n_splits, events,
                     f32_scores)


def mla8_batch(kv_codes, kv_scales, t_rows: int, lc: int, rc: int, q_lat, q_rope, pos0: int,
               sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True,
               n_splits: int = 0, events=None, f32_scores: bool = False,
               _fn: str = "mla8_batch"):
    """Causal batch: q [S, H, *]; query s attends rows [0, pos0 + s]."""
    mixed = _fn == "mla8_batch_mx"
    cap = _shadow(kv_codes, kv_scales, lc + (2 if mixed else 1) * rc)
    dev = kv_codes.device
    if not (1 <= int(t_rows) <= cap):
        raise ValueError(f"mla8: t_rows = {t_rows} outside the shadow's [1, {cap}] rows")
    _dev(q_lat, "q_lat", torch.float32, (None, None, lc), dev)
    n_q, h = q_lat.shape[0], q_lat.shape[1]
    _queries(q_lat, q_rope, (n_q, h), lc, rc, dev)
    out, lse = _out_lse(out, lse, (n_q, h), lc, dev, want_lse)
    ws = _workspace(MLA8_OP_BATCH, pos0 + n_q, h, n_q, lc, dev, workspace, n_splits)
    o = _opts(n_splits, events, f32_scores)
    _check(getattr(lib, _fn)(_ptr(kv_codes), _ptr(kv_scales), t_rows, lc, rc, _ptr(q_lat),
                             _ptr(q_rope), n_q, pos0, h, float(sm_scale), _ptr(out), _ptr(lse),
                             _ptr(ws), ws.numel(), _stream(q_lat), _o(o)), _fn)
    return out, lse


def mla8_batch_mx(kv_rows, kv_scales, t_rows: int, lc: int, rc: int, q_lat, q_rope, pos0: int,
                  sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True,
                  n_splits: int = 0, events=None, f32_scores: bool = False):
    """As mla8_batch over mixed rows."""
    return mla8_batch(kv_rows, kv_scales, t_rows, lc, rc, q_lat, q_rope, pos0, sm_scale, out, lse,
                      workspace, want_lse, n_splits, events, f32_scores, _fn="mla8_batch_mx")


# ---------------------------------------------------------------------------
# indexer

def mla8_index_topk(k_codes, k_scales, q, w, top_k: int, sel=None, scores=None,
                    workspace=None, want_scores: bool = False, events=None):
    """fp8 indexer score + top-k over key rows k_codes [T, 128] (e4m3) with
    scales [T]; q [n_ih, 128] f32, w [n_ih] f32.  Returns (sel int32
    [min(top_k, T)] ascending, scores f32 [T] or None)."""
    _dev(k_codes, "k_codes", torch.uint8, (None, None))
    t, ihd = k_codes.shape
    dev = k_codes.device
    _dev(k_scales, "k_scales", torch.float32, (t,), dev)
    _dev(q, "q", torch.float32, (None, ihd), dev)
    n_ih = q.shape[0]
    _dev(w, "w", torch.float32, (n_ih,), dev)
    if top_k < 1:
        raise ValueError("mla8: top_k must be >= 1")
    if sel is None:
        sel = torch.empty((min(top_k, t),), dtype=torch.int32, device=dev)
    _dev(sel, "sel", torch.int32, (min(top_k, t),), dev)
    if scores is None and want_scores:
        scores = torch.empty((t,), dtype=torch.float32, device=dev)
    elif scores is not None:
        _dev(scores, "scores", torch.float32, (t,), dev)
    need = mla8_workspace_bytes(MLA8_OP_INDEX, t, n_ih, 1, ihd)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, (None,), dev)
    o = _opts(0, events)
    _check(lib.mla8_index_topk(_ptr(k_codes), _ptr(k_scales), t, ihd, _ptr(q), _ptr(w), n_ih,
                               top_k, _ptr(sel), _ptr(scores), _ptr(workspace),
                               workspace.numel(), _stream(q), _o(o)), "mla8_index_topk")
    return sel, scores


# ---------------------------------------------------------------------------
# persistent shadow files

def _mem_ptr(t) -> int:
    """Address of a torch tensor (either device) or a numpy array."""
    if isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise ValueError("mla8: shadow tensors must be contiguous")
        return t.data_ptr()
    if not t.flags["C_CONTIGUOUS"]:
        raise ValueError("mla8: shadow arrays must be C-contiguous")
    return t.ctypes.data


def _ptr_table(ts):
    return (ctypes.c_void_p * len(ts))(*[_mem_ptr(t) for t in ts])


def _on_device(t) -> bool:
    return isinstance(t, torch.Tensor) and t.is_cuda


def _file_shadows(codes, scales, row_bytes: int):
    """Per-layer shadows for the file calls: all on the device or all on the
    host, [cap, row_bytes] bytes and [cap] f32 scales, one cap for all."""
    if len(codes) != len(scales) or len(codes) == 0:
        raise ValueError("mla8: codes and scales must be non-empty lists of equal length")
    dev = _on_device(codes[0])
    cap = codes[0].shape[0]
    for c, s in zip(codes, scales):
        if _on_device(c) != dev or _on_device(s) != dev:
            raise ValueError("mla8: shadows must all be device tensors or all host arrays")
        if tuple(c.shape) != (cap, row_bytes) or tuple(s.shape) != (cap,):
            raise ValueError(f"mla8: shadow shapes must be [{cap}, {row_bytes}] and [{cap}]")
        if str(c.dtype) not in ("torch.uint8", "uint8") or \
                str(s.dtype) not in ("torch.float32", "float32"):
            raise ValueError("mla8: shadow codes must be uint8 and scales float32")
    return dev, cap


def mla8_kvfile_create(path: str, n_layers: int, lc: int, rc: int) -> None:
    _check(lib.mla8_kvfile_create(os.fsencode(path), n_layers, lc, rc), "mla8_kvfile_create")


def mla8_kvfile_info(path: str) -> dict:
    v, nl, lc, rc = (ctypes.c_int32() for _ in range(4))
    nt = ctypes.c_int64()
    _check(lib.mla8_kvfile_info(os.fsencode(path), ctypes.byref(v), ctypes.byref(nl),
                                ctypes.byref(lc), ctypes.byref(rc), ctypes.byref(nt)),
           "mla8_kvfile_info")
    return {"version": v.value, "n_layers": nl.value, "lc": lc.value, "rc": rc.value,
            "n_tokens": nt.value}


def mla8_kvfile_append(path: str, codes, scales, t0: int, n_tok: int, lc: int, rc: int) -> None:
    """Append rows [t0, t0 + n_tok) of every layer's shadow (lists of device
    tensors, or of host arrays) to the file."""
    dev, cap = _file_shadows(codes, scales, lc + rc)
    if t0 < 0 or n_tok < 0 or t0 + n_tok > cap:
        raise ValueError(f"mla8: rows [{t0}, {t0 + n_tok}) outside the shadows' {cap} rows")
    _check(lib.mla8_kvfile_append(os.fsencode(path), len(codes), _ptr_table(codes),
                                  _ptr_table(scales), t0, n_tok, lc, rc, int(dev),
                                  _stream(codes[0]) if dev else None), "mla8_kvfile_append")


def mla8_kvfile_load(path: str, codes, scales, lc: int, rc: int, workspace=None) -> int:
    """Load the file's committed tokens into every layer's shadow; returns t_rows."""
    dev, cap = _file_shadows(codes, scales, lc + rc)
    t = ctypes.c_int64(0)
    ws_ptr, ws_n = None, 0
    if workspace is not None:
        if dev:
            _dev(workspace, "workspace", workspace.dtype, None, codes[0].device)
        ws_ptr, ws_n = _mem_ptr(workspace), workspace.numel() * workspace.element_size()
    _check(lib.mla8_kvfile_load(os.fsencode(path), len(codes), _ptr_table(codes),
                                _ptr_table(scales), cap, ctypes.byref(t), lc, rc,
                                int(dev), ws_ptr, ws_n, _stream(codes[0]) if dev else None),
           "mla8_kvfile_load")
    return int(t.value)


# ---------------------------------------------------------------------------
# auxiliary calls (include/mla8_aux.h)

def mla8_stream_read(t: torch.Tensor, out: torch.Tensor) -> None:
    """Load every byte of the device tensor t once, XOR-folding its 32-bit
    words into out (int32 [MLA8_STREAM_WORDS] on the device, one fold per
    wave; their XOR is the buffer's): the read-bandwidth reference."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError("mla8_stream_read: t must be a contiguous device tensor")
    _dev(out, "out", out.dtype, None, t.device)
    if out.numel() * out.element_size() < 4 * MLA8_STREAM_WORDS:
        raise ValueError("mla8_stream_read: out needs MLA8_STREAM_WORDS 32-bit words")
    _check(lib.mla8_stream_read(_ptr(t), t.numel() * t.element_size(), _ptr(out), _stream(t)),
           "mla8_stream_read")


def mla8_test_encode(x: torch.Tensor, codes: torch.Tensor | None = None) -> torch.Tensor:
    """Device e4m3 encoder applied elementwise (test aid, not product API)."""
    _dev(x, "x", torch.float32)
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _dev(codes, "codes", torch.uint8, tuple(x.shape), x.device)
    _check(lib.mla8_test_encode(_ptr(x), x.numel(), _ptr(codes), _stream(x)), "mla8_test_encode")
    return codes


def mla8_test_encode_pk(x: torch.Tensor, codes: torch.Tensor | None = None) -> torch.Tensor:
    """The packed hardware e4m3 encoder of the query's lo term, elementwise
    (test aid, not product API; exact for finite |x| < 448).  x.numel() a
    multiple of 4."""
    _dev(x, "x", torch.float32)
    if x.numel() % 4 != 0:
        raise ValueError("mla8_test_encode_pk: x.numel() must be a multiple of 4")
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _dev(codes, "codes", torch.uint8, tuple(x.shape), x.device)
    _check(lib.mla8_test_encode_pk(_ptr(x), x.numel(), _ptr(codes), _stream(x)),
           "mla8_test_encode_pk")
    return codes
