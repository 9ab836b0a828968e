"""Thin Python binding over libmla8.so (include/mla8.h), same names as the C ABI.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels.  The
library must be built (``python -m fp8_mla_latent_amd.build``); importing this
module without it raises, there is no fallback path.
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
MLA8_OP_DECODE = 0
MLA8_OP_DECODE_SEL = 1
MLA8_OP_BATCH = 2
MLA8_OP_INDEX = 3

EXPORTED = ("mla8_quantize_rows", "mla8_append", "mla8_decode", "mla8_append_decode",
            "mla8_decode_sel", "mla8_batch", "mla8_quantize_rows_mx", "mla8_append_mx",
            "mla8_decode_mx", "mla8_decode_sel_mx", "mla8_append_decode_mx", "mla8_batch_mx",
            "mla8_index_topk", "mla8_kvfile_create",
            "mla8_kvfile_info", "mla8_kvfile_append", "mla8_kvfile_load",
            "mla8_workspace_bytes", "mla8_force_splits", "mla8_plan_splits",
            "mla8_status_string", "mla8_version", "mla8_test_encode", "mla8_profile_events",
            "mla8_stream_read")


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
    sig = {
        "mla8_quantize_rows": (ctypes.c_int, [P, i64, i32, i32, P, P, P]),
        "mla8_append": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64, i32, i32, P]),
        "mla8_decode": (ctypes.c_int, [P, P, i64, i32, i32, P, P, i32, f32, P, P, P, sz, P]),
        "mla8_append_decode": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64, i32, i32,
                                              P, P, i32, f32, P, P, P, sz, P]),
        "mla8_decode_sel": (ctypes.c_int,
                            [P, P, i64, i32, i32, P, i64, P, P, i32, f32, P, P, P, sz, P]),
        "mla8_batch": (ctypes.c_int,
                       [P, P, i64, i32, i32, P, P, i32, i64, i32, f32, P, P, P, sz, P]),
        "mla8_quantize_rows_mx": (ctypes.c_int, [P, i64, i32, i32, P, P, P]),
        "mla8_append_mx": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64, i32, i32, P]),
        "mla8_decode_mx": (ctypes.c_int, [P, P, i64, i32, i32, P, P, i32, f32, P, P, P, sz, P]),
        "mla8_decode_sel_mx": (ctypes.c_int,
                               [P, P, i64, i32, i32, P, i64, P, P, i32, f32, P, P, P, sz, P]),
        "mla8_append_decode_mx": (ctypes.c_int, [P, P, i64, ctypes.POINTER(i64), P, i64, i32,
                                                 i32, P, P, i32, f32, P, P, P, sz, P]),
        "mla8_batch_mx": (ctypes.c_int,
                          [P, P, i64, i32, i32, P, P, i32, i64, i32, f32, P, P, P, sz, P]),
        "mla8_index_topk": (ctypes.c_int,
                            [P, P, i64, i32, P, P, i32, i32, P, P, P, sz, P]),
        "mla8_kvfile_create": (ctypes.c_int, [ctypes.c_char_p, i32, i32, i32]),
        "mla8_kvfile_info": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(i32),
                                            ctypes.POINTER(i32), ctypes.POINTER(i32),
                                            ctypes.POINTER(i32), ctypes.POINTER(i64)]),
        "mla8_kvfile_append": (ctypes.c_int, [ctypes.c_char_p, i32, P, P, i64, i64, i32, i32,
                                              i32, P]),
        "mla8_kvfile_load": (ctypes.c_int, [ctypes.c_char_p, i32, P, P, i64,
                                            ctypes.POINTER(i64), i32, i32, i32, P, sz, P]),
        "mla8_workspace_bytes": (sz, [i32, i64, i32, i32, i32]),
        "mla8_force_splits": (i32, [i32]),
        "mla8_plan_splits": (i32, [i32, i64, i32, i32]),
        "mla8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "mla8_version": (ctypes.c_char_p, []),
        "mla8_test_encode": (ctypes.c_int, [P, i64, P, P]),
        "mla8_stream_read": (ctypes.c_int, [P, i64, P, P]),
        "mla8_profile_events": (ctypes.c_int, [P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


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


def mla8_status_string(status: int) -> str:
    return lib.mla8_status_string(status).decode()


def mla8_version() -> str:
    return lib.mla8_version().decode()


def mla8_workspace_bytes(op: int, rows: int, n_heads: int, n_q: int, lc: int) -> int:
    return int(lib.mla8_workspace_bytes(op, rows, n_heads, n_q, lc))


def mla8_force_splits(n_splits: int) -> int:
    return int(lib.mla8_force_splits(n_splits))


def mla8_plan_splits(op: int, rows: int, n_heads: int, n_q: int = 1) -> int:
    return int(lib.mla8_plan_splits(op, rows, n_heads, n_q))


def _workspace(op, rows, n_heads, n_q, lc, device, workspace):
    need = mla8_workspace_bytes(op, rows, n_heads, n_q, lc)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace


def mla8_quantize_rows(x: torch.Tensor, lc: int, rc: int, codes: torch.Tensor | None = None,
                       scales: torch.Tensor | None = None):
    """f32 rows [n, lc+rc] -> (uint8 codes [n, lc+rc], f32 scales [n])."""
    n = x.shape[0]
    if codes is None:
        codes = torch.empty((n, lc + rc), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n,), dtype=torch.float32, device=x.device)
    _check(lib.mla8_quantize_rows(_ptr(x), n, lc, rc, _ptr(codes), _ptr(scales), _stream(x)),
           "mla8_quantize_rows")
    return codes, scales


def mla8_append(kv_codes: torch.Tensor, kv_scales: torch.Tensor, t_rows: int, x: torch.Tensor,
                lc: int, rc: int) -> int:
    """Quantize rows x into the shadow at [t_rows, t_rows + n); returns the new t_rows."""
    t = ctypes.c_int64(t_rows)
    _check(lib.mla8_append(_ptr(kv_codes), _ptr(kv_scales), kv_codes.shape[0], ctypes.byref(t),
                           _ptr(x), x.shape[0], lc, rc, _stream(x)), "mla8_append")
    return int(t.value)


def mla8_decode(kv_codes, kv_scales, t_rows: int, lc: int, rc: int, q_lat, q_rope,
                sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True):
    """Dense decode over shadow rows [0, t_rows): returns (out [H, lc], lse [H] or None)."""
    h = q_lat.shape[0]
    dev = q_lat.device
    if out is None:
        out = torch.empty((h, lc), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((h,), dtype=torch.float32, device=dev)
    ws = _workspace(MLA8_OP_DECODE, t_rows, h, 1, lc, dev, workspace)
    _check(lib.mla8_decode(_ptr(kv_codes), _ptr(kv_scales), t_rows, lc, rc, _ptr(q_lat),
                           _ptr(q_rope), h, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws),
                           ws.numel(), _stream(q_lat)), "mla8_decode")
    return out, lse


def mla8_append_decode(kv_codes, kv_scales, t_rows: int, x_new, lc: int, rc: int, q_lat, q_rope,
                       sm_scale: float, out=None, lse=None, workspace=None,
                       want_lse: bool = True, _fn: str = "mla8_append_decode"):
    """Append x_new [n, lc+rc] at rows [t_rows, t_rows + n) and decode over all
    t_rows + n rows in one launch: returns (out, lse, new t_rows)."""
    h = q_lat.shape[0]
    dev = q_lat.device
    n = x_new.shape[0]
    if out is None:
        out = torch.empty((h, lc), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((h,), dtype=torch.float32, device=dev)
    ws = _workspace(MLA8_OP_DECODE, t_rows + n, h, 1, lc, dev, workspace)
    t = ctypes.c_int64(t_rows)
    _check(getattr(lib, _fn)(_ptr(kv_codes), _ptr(kv_scales), kv_codes.shape[0],
                             ctypes.byref(t), _ptr(x_new), n, lc, rc, _ptr(q_lat),
                             _ptr(q_rope), h, float(sm_scale), _ptr(out), _ptr(lse),
                             _ptr(ws), ws.numel(), _stream(q_lat)), _fn)
    return out, lse, int(t.value)


def mla8_append_decode_mx(kv_rows, kv_scales, t_rows: int, x_new, lc: int, rc: int, q_lat,
                          q_rope, sm_scale: float, out=None, lse=None, workspace=None,
                          want_lse: bool = True):
    """As mla8_append_decode over mixed rows (kv_rows [cap, lc + 2 rc])."""
    return mla8_append_decode(kv_rows, kv_scales, t_rows, x_new, lc, rc, q_lat, q_rope, sm_scale,
                              out, lse, workspace, want_lse, _fn="mla8_append_decode_mx")


def mla8_decode_sel(kv_codes, kv_scales, t_rows: int, lc: int, rc: int, sel, q_lat, q_rope,
                    sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True):
    """Decode over the selected absolute rows sel [ns] (int32)."""
    h = q_lat.shape[0]
    dev = q_lat.device
    ns = sel.numel()
    if out is None:
        out = torch.empty((h, lc), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((h,), dtype=torch.float32, device=dev)
    ws = _workspace(MLA8_OP_DECODE_SEL, ns, h, 1, lc, dev, workspace)
    _check(lib.mla8_decode_sel(_ptr(kv_codes), _ptr(kv_scales), t_rows, lc, rc, _ptr(sel), ns,
                               _ptr(q_lat), _ptr(q_rope), h, float(sm_scale), _ptr(out),
                               _ptr(lse), _ptr(ws), ws.numel(), _stream(q_lat)),
           "mla8_decode_sel")
    return out, lse


def mla8_batch(kv_codes, kv_scales, t_rows: int, lc: int, rc: int, q_lat, q_rope, pos0: int,
               sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True,
               _fn: str = "mla8_batch"):
    """Causal batch: q [S, H, *]; query s attends rows [0, pos0 + s]."""
    n_q, h = q_lat.shape[0], q_lat.shape[1]
    dev = q_lat.device
    if out is None:
        out = torch.empty((n_q, h, lc), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((n_q, h), dtype=torch.float32, device=dev)
    ws = _workspace(MLA8_OP_BATCH, pos0 + n_q, h, n_q, lc, dev, workspace)
    _check(getattr(lib, _fn)(_ptr(kv_codes), _ptr(kv_scales), t_rows, lc, rc, _ptr(q_lat),
                             _ptr(q_rope), n_q, pos0, h, float(sm_scale), _ptr(out), _ptr(lse),
                             _ptr(ws), ws.numel(), _stream(q_lat)), _fn)
    return out, lse


def mla8_batch_mx(kv_rows, kv_scales, t_rows: int, lc: int, rc: int, q_lat, q_rope, pos0: int,
                  sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True):
    """As mla8_batch over mixed rows."""
    return mla8_batch(kv_rows, kv_scales, t_rows, lc, rc, q_lat, q_rope, pos0, sm_scale, out, lse,
                      workspace, want_lse, _fn="mla8_batch_mx")


def mla8_quantize_rows_mx(x: torch.Tensor, lc: int, rc: int, rows=None, scales=None):
    """Mixed rows: f32 [n, lc + rc] -> (uint8 rows [n, lc + 2 rc], f32 scales [n])."""
    n = x.shape[0]
    if rows is None:
        rows = torch.empty((n, lc + 2 * rc), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n,), dtype=torch.float32, device=x.device)
    _check(lib.mla8_quantize_rows_mx(_ptr(x), n, lc, rc, _ptr(rows), _ptr(scales), _stream(x)),
           "mla8_quantize_rows_mx")
    return rows, scales


def mla8_append_mx(kv_rows, kv_scales, t_rows: int, x, lc: int, rc: int) -> int:
    t = ctypes.c_int64(t_rows)
    _check(lib.mla8_append_mx(_ptr(kv_rows), _ptr(kv_scales), kv_rows.shape[0], ctypes.byref(t),
                              _ptr(x), x.shape[0], lc, rc, _stream(x)), "mla8_append_mx")
    return int(t.value)


def mla8_decode_mx(kv_rows, kv_scales, t_rows: int, lc: int, rc: int, q_lat, q_rope,
                   sm_scale: float, out=None, lse=None, workspace=None, want_lse: bool = True):
    """Dense decode over mixed rows [0, t_rows): (out [H, lc], lse [H] or None)."""
    h = q_lat.shape[0]
    dev = q_lat.device
    if out is None:
        out = torch.empty((h, lc), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((h,), dtype=torch.float32, device=dev)
    ws = _workspace(MLA8_OP_DECODE, t_rows, h, 1, lc, dev, workspace)
    _check(lib.mla8_decode_mx(_ptr(kv_rows), _ptr(kv_scales), t_rows, lc, rc, _ptr(q_lat),
                              _ptr(q_rope), h, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws),
                              ws.numel(), _stream(q_lat)), "mla8_decode_mx")
    return out, lse


def mla8_decode_sel_mx(kv_rows, kv_scales, t_rows: int, lc: int, rc: int, sel, q_lat, q_rope,
                       sm_scale: float, out=None, lse=None, workspace=None,
                       want_lse: bool = True):
    """Decode over the selected mixed rows sel (int32 device tensor)."""
    h = q_lat.shape[0]
    dev = q_lat.device
    ns = sel.shape[0]
    if out is None:
        out = torch.empty((h, lc), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((h,), dtype=torch.float32, device=dev)
    ws = _workspace(MLA8_OP_DECODE_SEL, ns, h, 1, lc, dev, workspace)
    _check(lib.mla8_decode_sel_mx(_ptr(kv_rows), _ptr(kv_scales), t_rows, lc, rc, _ptr(sel), ns,
                                  _ptr(q_lat), _ptr(q_rope), h, float(sm_scale), _ptr(out),
                                  _ptr(lse), _ptr(ws), ws.numel(), _stream(q_lat)),
           "mla8_decode_sel_mx")
    return out, lse


def mla8_index_topk(k_codes, k_scales, q, w, top_k: int, sel=None, scores=None,
                    workspace=None, want_scores: bool = False):
    """fp8 indexer score + top-k over key rows k_codes [T, 128] (e4m3) with
    scales [T]; q [n_ih, 128] f32, w [n_ih] f32.  Returns (sel int32
    [min(top_k, T)] ascending, scores f32 [T] or None)."""
    t, ihd = k_codes.shape
    n_ih = q.shape[0]
    dev = q.device
    if sel is None:
        sel = torch.empty((min(top_k, t),), dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        scores = torch.empty((t,), dtype=torch.float32, device=dev)
    if workspace is None:
        need = mla8_workspace_bytes(MLA8_OP_INDEX, t, n_ih, 1, ihd)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.mla8_index_topk(_ptr(k_codes), _ptr(k_scales), t, ihd, _ptr(q), _ptr(w), n_ih,
                               top_k, _ptr(sel), _ptr(scores), _ptr(workspace),
                               workspace.numel(), _stream(q)), "mla8_index_topk")
    return sel, scores


def _mem_ptr(t) -> int:
    """Address of a torch tensor (either device) or a numpy array."""
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    return t.ctypes.data


def _ptr_table(ts):
    return (ctypes.c_void_p * len(ts))(*[_mem_ptr(t) for t in ts])


def _on_device(t) -> bool:
    return isinstance(t, torch.Tensor) and t.is_cuda


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
    dev = _on_device(codes[0])
    _check(lib.mla8_kvfile_append(os.fsencode(path), len(codes), _ptr_table(codes),
                                  _ptr_table(scales), t0, n_tok, lc, rc, int(dev),
                                  _stream(codes[0]) if dev else None), "mla8_kvfile_append")


def mla8_kvfile_load(path: str, codes, scales, lc: int, rc: int, workspace=None) -> int:
    """Load the file's committed tokens into every layer's shadow; returns t_rows."""
    dev = _on_device(codes[0])
    t = ctypes.c_int64(0)
    ws_ptr, ws_n = None, 0
    if workspace is not None:
        ws_ptr, ws_n = _mem_ptr(workspace), workspace.numel()
    _check(lib.mla8_kvfile_load(os.fsencode(path), len(codes), _ptr_table(codes),
                                _ptr_table(scales), codes[0].shape[0], ctypes.byref(t), lc, rc,
                                int(dev), ws_ptr, ws_n, _stream(codes[0]) if dev else None),
           "mla8_kvfile_load")
    return int(t.value)


def mla8_profile_events(before: "torch.cuda.Event | None", after: "torch.cuda.Event | None"):
    """Record `before`/`after` around the split-T partial kernel of the next
    attention calls (None, None clears).  torch creates an event's hipEvent on
    its first record(), so record both once before passing them."""
    def raw(ev):
        if ev is None:
            return None
        if not ev.cuda_event:
            raise ValueError("mla8_profile_events: record the event once first")
        return ev.cuda_event
    _check(lib.mla8_profile_events(raw(before), raw(after)), "mla8_profile_events")


MLA8_STREAM_WORDS = 32768


def mla8_stream_read(t: torch.Tensor, out: torch.Tensor) -> None:
    """Load every byte of the device tensor t once, XOR-folding its 32-bit
    words into out (int32 [MLA8_STREAM_WORDS] on the device, one fold per
    wave; their XOR is the buffer's): the read-bandwidth reference."""
    if out.numel() * out.element_size() < 4 * MLA8_STREAM_WORDS:
        raise ValueError("mla8_stream_read: out needs MLA8_STREAM_WORDS 32-bit words")
    _check(lib.mla8_stream_read(_ptr(t), t.numel() * t.element_size(), _ptr(out), _stream(t)),
           "mla8_stream_read")


def mla8_test_encode(x: torch.Tensor, codes: torch.Tensor | None = None) -> torch.Tensor:
    """Device e4m3 encoder applied elementwise (test hook, not product API)."""
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib.mla8_test_encode(_ptr(x), x.numel(), _ptr(codes), _stream(x)), "mla8_test_encode")
    return codes
