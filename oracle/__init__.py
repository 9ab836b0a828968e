"""mla8 oracle -- TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes wrapper over ``mla8_oracle.c``, the plain double-precision CPU
implementation of the fp8 latent-KV MLA decode path.  Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import this package; the
product library never does.  Nothing here shares code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: every f32 product and quotient in the quantizer is rounded
# on its own, as the definition states; -fno-fast-math keeps IEEE semantics.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.mla8o_dec.restype = ctypes.c_double
        L.mla8o_dec.argtypes = [ctypes.c_uint8]
        L.mla8o_enc.restype = ctypes.c_uint8
        L.mla8o_enc.argtypes = [f32]
        L.mla8o_encode_array.argtypes = [P, i64, P]
        L.mla8o_decode_array.argtypes = [P, i64, P]
        L.mla8o_quantize_row.argtypes = [P, i32, P, P]
        L.mla8o_quantize_rows.argtypes = [P, i64, i32, P, P]
        L.mla8o_decode.argtypes = [P, P, i64, i32, i32, P, P, i32, f32, P, P]
        L.mla8o_decode_sel.argtypes = [P, P, i64, i32, i32, P, i64, P, P, i32, f32, P, P]
        L.mla8o_batch.argtypes = [P, P, i64, i32, i32, P, P, i32, i64, i32, f32, P, P]
        L.mla8o_decode_chunked.argtypes = [P, P, i64, i32, i32, P, P, i32, f32, i64, P, P]
        L.mla8o_index_scores.argtypes = [P, P, i64, i32, P, P, i32, P]
        L.mla8o_bf16.restype = ctypes.c_uint16
        L.mla8o_bf16.argtypes = [f32]
        L.mla8o_bf16_array.argtypes = [P, i64, P]
        L.mla8o_bf16_value.restype = ctypes.c_double
        L.mla8o_bf16_value.argtypes = [ctypes.c_uint16]
        L.mla8o_quantize_rows_mx.argtypes = [P, i64, i32, i32, P, P]
        L.mla8o_decode_mx.argtypes = [P, P, i64, i32, i32, P, P, i32, f32, P, P]
        L.mla8o_decode_sel_mx.argtypes = [P, P, i64, i32, i32, P, i64, P, P, i32, f32, P, P]
        L.mla8o_threads.restype = ctypes.c_int
        L.mla8o_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def dec(codes) -> np.ndarray:
    """e4m3 bytes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().mla8o_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def enc(x) -> np.ndarray:
    """float32 values -> e4m3 bytes (RNE, saturating, NaN -> 0x00)."""
    v = _c(x, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().mla8o_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """f32 rows [n, D] -> (e4m3 codes [n, D] uint8, f32 scales [n])."""
    v = _c(x, np.float32)
    n, d = v.shape
    codes = np.empty((n, d), np.uint8)
    scales = np.empty((n,), np.float32)
    lib().mla8o_quantize_rows(_ptr(v), n, d, _ptr(codes), _ptr(scales))
    return codes, scales


def dequant(codes, scales) -> np.ndarray:
    """Exact float64 values of a quantized shadow: dec(code) * scale."""
    return dec(codes) * np.asarray(scales, np.float64)[..., None]


def decode(codes, scales, t_rows, lc, rc, q_lat, q_rope, sm_scale):
    """Dense decode of H heads over rows [0, t_rows): (out [H, lc] f64, lse [H] f64)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    ql = _c(q_lat, np.float32)
    qr = _c(q_rope, np.float32)
    h = ql.shape[0]
    out = np.empty((h, lc), np.float64)
    lse = np.empty((h,), np.float64)
    lib().mla8o_decode(_ptr(codes), _ptr(scales), t_rows, lc, rc, _ptr(ql), _ptr(qr), h,
                       float(np.float32(sm_scale)), _ptr(out), _ptr(lse))
    return out, lse


def decode_sel(codes, scales, t_rows, lc, rc, sel, q_lat, q_rope, sm_scale):
    """Decode over the selected absolute rows ``sel`` (a multiset; out-of-range skipped)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    s = _c(sel, np.int32)
    ql = _c(q_lat, np.float32)
    qr = _c(q_rope, np.float32)
    h = ql.shape[0]
    out = np.empty((h, lc), np.float64)
    lse = np.empty((h,), np.float64)
    lib().mla8o_decode_sel(_ptr(codes), _ptr(scales), t_rows, lc, rc, _ptr(s), s.size,
                           _ptr(ql), _ptr(qr), h, float(np.float32(sm_scale)), _ptr(out),
                           _ptr(lse))
    return out, lse


def batch(codes, scales, t_rows, lc, rc, q_lat, q_rope, pos0, sm_scale):
    """Causal batch: query s (position pos0+s) attends rows [0, pos0+s]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    ql = _c(q_lat, np.float32)
    qr = _c(q_rope, np.float32)
    n_q, h = ql.shape[0], ql.shape[1]
    out = np.empty((n_q, h, lc), np.float64)
    lse = np.empty((n_q, h), np.float64)
    lib().mla8o_batch(_ptr(codes), _ptr(scales), t_rows, lc, rc, _ptr(ql), _ptr(qr), n_q,
                      pos0, h, float(np.float32(sm_scale)), _ptr(out), _ptr(lse))
    return out, lse


def decode_chunked(codes, scales, t_rows, lc, rc, q_lat, q_rope, sm_scale, n_chunks):
    """Split-T decode: per-chunk streaming partials + log-sum-exp merge."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    ql = _c(q_lat, np.float32)
    qr = _c(q_rope, np.float32)
    h = ql.shape[0]
    out = np.empty((h, lc), np.float64)
    lse = np.empty((h,), np.float64)
    lib().mla8o_decode_chunked(_ptr(codes), _ptr(scales), t_rows, lc, rc, _ptr(ql), _ptr(qr),
                               h, float(np.float32(sm_scale)), n_chunks, _ptr(out), _ptr(lse))
    return out, lse


def index_scores(k_codes, k_scales, q, w):
    """Indexer scores I_t [T] f64 of one query token: q [n_ih, ihd] f32 (quantized
    per head inside), w [n_ih] f32, keys e4m3 [T, ihd] with f32 scales [T]."""
    kc = _c(k_codes, np.uint8)
    ks = _c(k_scales, np.float32)
    qq = _c(q, np.float32)
    ww = _c(w, np.float32)
    t, ihd = kc.shape
    n_ih = qq.shape[0]
    assert qq.shape == (n_ih, ihd) and ww.shape == (n_ih,) and ks.shape == (t,)
    out = np.empty((t,), np.float64)
    lib().mla8o_index_scores(_ptr(kc), _ptr(ks), t, ihd, _ptr(qq), _ptr(ww), n_ih, _ptr(out))
    return out


def index_topk(scores, top_k):
    """[B2-indexer] top-k: the min(top_k, T) rows with the largest scores, ties
    to the smaller row index, a NaN score below every other; returned as row
    indices in ascending order (int32)."""
    s = np.asarray(scores, np.float64)
    t = np.arange(s.size)
    nan = np.isnan(s)
    neg = np.where(nan, 0.0, -s)
    # sort keys, last is primary: NaN class, then score descending, then row
    order = np.lexsort((t, neg, nan.astype(np.int8)))
    return np.sort(order[:min(int(top_k), s.size)]).astype(np.int32)


def bf16(x) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even."""
    v = _c(np.asarray(x, np.float32).ravel(), np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().mla8o_bf16_array(_ptr(v), v.size, _ptr(out))
    return out.reshape(np.shape(x))


def bf16_value(b) -> np.ndarray:
    """bf16 bit patterns -> float64 values."""
    v = np.asarray(b, np.uint16).ravel()
    f = lib().mla8o_bf16_value
    return np.array([f(int(t)) for t in v], np.float64).reshape(np.shape(b))


def query_lo8_mx(q_lat, q_rope, sm_scale):
    """The query that the mixed-row decode (noPE e4m3 + RoPE bf16) attends
    with by default (mla8_opts.f32_scores turns it off): the query_lo8
    construction on the noPE part alone, and the RoPE part as two bf16 terms.

    Reading of [B1-FMHA first pass, intentional first-pass limits: the noPE QK
    product on the fp8 tensor cores; RoPE stays bf16] on this library's terms.
    es = f32(sm_scale) * f32(log2 e) (an f32 product).  noPE, per head: k = 15
    - ex(f32(max|q_lat| * es)) capped at 100 (0 for a zero head), r =
    f32(q_lat * f32(es 2^k)), hi = fp16(r), lo = fp16(r - hi), j = 8 -
    ex(max|lo|) clamped to [-100, 100] (0 when lo is all zero), lo8 =
    enc(f32(lo 2^j)); q_lat' = (hi + dec(lo8) 2^-j) 2^-k / es.  The RoPE part
    does not enter k.  RoPE, per element: e = f32(q_rope * es), hi = bf16(e),
    lo = bf16(f32(e - hi)) (round to nearest even); q_rope' = (hi + lo) / es.
    Returns (q_lat' [H, lc], q_rope' [H, rc]) as float32 arrays.
    """
    ql = np.asarray(q_lat, np.float32)
    qr = np.asarray(q_rope, np.float32)
    es = np.float32(np.float32(sm_scale) * np.float32(1.4426950408889634))
    out_l = np.empty(ql.shape, np.float64)
    for h in range(ql.shape[0]):
        e = ql[h]
        emax = np.float32(np.max(np.abs(e)) * es) if e.size else np.float32(0)
        k = min(15 - int(np.frexp(emax)[1]), 100) if emax > 0 else 0
        mult = np.float32(np.ldexp(es, k))
        r = (e * mult).astype(np.float32)
        hi = r.astype(np.float16)
        lo = (r - hi.astype(np.float32)).astype(np.float16)
        lmax = float(np.max(np.abs(lo.astype(np.float32)))) if lo.size else 0.0
        j = max(-100, min(100, 8 - int(np.frexp(lmax)[1]))) if lmax > 0 else 0
        lo8 = enc(np.ldexp(lo.astype(np.float32), j).astype(np.float32))
        out_l[h] = np.ldexp(hi.astype(np.float64) + np.ldexp(dec(lo8), -j), -k) / np.float64(es)
    e = (qr * es).astype(np.float32)
    rhi = bf16(e)
    rhi_v = bf16_value(rhi)
    rlo = bf16((e.astype(np.float64) - rhi_v).astype(np.float32))
    out_r = (rhi_v + bf16_value(rlo)) / np.float64(es)
    return (np.ascontiguousarray(out_l.astype(np.float32)),
            np.ascontiguousarray(out_r.astype(np.float32)))


def quantize_rows_mx(x, lc, rc) -> tuple[np.ndarray, np.ndarray]:
    """Mixed rows: f32 [n, lc + rc] -> (rows uint8 [n, lc + 2 rc], scales f32 [n])."""
    v = _c(x, np.float32)
    n = v.shape[0]
    assert v.shape[1] == lc + rc
    rows = np.empty((n, lc + 2 * rc), np.uint8)
    scales = np.empty((n,), np.float32)
    lib().mla8o_quantize_rows_mx(_ptr(v), n, lc, rc, _ptr(rows), _ptr(scales))
    return rows, scales


def decode_mx(rows, scales, t_rows, lc, rc, q_lat, q_rope, sm_scale):
    """Dense decode of H heads over mixed rows [0, t_rows)."""
    r = _c(rows, np.uint8)
    sc = _c(scales, np.float32)
    ql = _c(q_lat, np.float32)
    qr = _c(q_rope, np.float32)
    h = ql.shape[0]
    out = np.empty((h, lc), np.float64)
    lse = np.empty((h,), np.float64)
    lib().mla8o_decode_mx(_ptr(r), _ptr(sc), t_rows, lc, rc, _ptr(ql), _ptr(qr), h,
                          float(np.float32(sm_scale)), _ptr(out), _ptr(lse))
    return out, lse


def decode_sel_mx(rows, scales, t_rows, lc, rc, sel, q_lat, q_rope, sm_scale):
    """Selected-row decode over mixed rows (a multiset; out-of-range skipped)."""
    r = _c(rows, np.uint8)
    sc = _c(scales, np.float32)
    s = _c(sel, np.int32)
    ql = _c(q_lat, np.float32)
    qr = _c(q_rope, np.float32)
    h = ql.shape[0]
    out = np.empty((h, lc), np.float64)
    lse = np.empty((h,), np.float64)
    lib().mla8o_decode_sel_mx(_ptr(r), _ptr(sc), t_rows, lc, rc, _ptr(s), s.size, _ptr(ql),
                              _ptr(qr), h, float(np.float32(sm_scale)), _ptr(out), _ptr(lse))
    return out, lse


def threads() -> int:
    return int(lib().mla8o_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for the following calls; n < 1 restores the default."""
    lib().mla8o_set_threads(int(n))


def query_lo8(q_lat, q_rope, sm_scale):
    """The query that the e4m3 512/64 decode attends with by default (its
    scores' lo term on the e4m3 MFMA; mla8_opts.f32_scores turns it off).

    Reading of [B1-FMHA first pass, intentional first-pass limits: the noPE QK
    product on the fp8 tensor cores] on this library's terms: the query stays
    f32 at the boundary; per head, e = q * es with es = f32(sm_scale) *
    f32(log2 e) (an f32 product) is scaled by 2^k, k = 15 - ex(f32(max|q| *
    es)) capped at 100 (0 for a zero head; ex is frexp's exponent), into r =
    f32(q * f32(es 2^k)); hi = fp16(r) (round to nearest even), lo = fp16(r -
    hi) (the difference is exact in f32); lo is quantized to e4m3 with the
    power-of-2 scale 2^j, j = 8 - ex(max|lo|) clamped to [-100, 100] (0 when
    lo is all zero): lo8 = enc(f32(lo 2^j)).  The scores are then
    sum_i x_i (hi_i + dec(lo8_i) 2^-j) 2^-k in log2 units, i.e. the dense
    attention of the query q' = (hi + dec(lo8) 2^-j) 2^-k / es, returned
    rounded to f32 (2^-24 relative, far below what the quantization moves).
    Returns (q_lat' [H, lc], q_rope' [H, rc]) as float32 arrays.
    """
    ql = np.asarray(q_lat, np.float32)
    qr = np.asarray(q_rope, np.float32)
    lc = ql.shape[1]
    q = np.concatenate([ql, qr], axis=1)
    es = np.float32(np.float32(sm_scale) * np.float32(1.4426950408889634))
    out = np.empty(q.shape, np.float64)
    for h in range(q.shape[0]):
        e = q[h]
        emax = np.float32(np.max(np.abs(e)) * es)
        k = min(15 - int(np.frexp(emax)[1]), 100) if emax > 0 else 0
        mult = np.float32(np.ldexp(es, k))
        r = (e * mult).astype(np.float32)
        hi = r.astype(np.float16)
        lo = (r - hi.astype(np.float32)).astype(np.float16)
        lmax = float(np.max(np.abs(lo.astype(np.float32))))
        j = max(-100, min(100, 8 - int(np.frexp(lmax)[1]))) if lmax > 0 else 0
        lo8 = enc(np.ldexp(lo.astype(np.float32), j).astype(np.float32))
        term = hi.astype(np.float64) + np.ldexp(dec(lo8), -j)
        out[h] = np.ldexp(term, -k) / np.float64(es)
    out32 = out.astype(np.float32)
    return np.ascontiguousarray(out32[:, :lc]), np.ascontiguousarray(out32[:, lc:])
