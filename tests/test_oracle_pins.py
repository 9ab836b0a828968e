"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: values the
source pages fix (golden anchors), a library routine on its sub-domain (torch's
float8_e4m3fn), an independent brute-force definition, closed forms and
invariants of softmax attention, or long-double brute force on tiny inputs.
The page passages are those of colibri PR #300 ("KV8 long-context CUDA: fp8
device shadow, split-T kernels, DSA-aware gather"): the KV8-base commit's
c/kv_fp8.h and attention_rows bullets, and the second commit's split-T and DSA
bullets.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.brute import MAGS, encode_bruteforce, half_gap, torch_decode_table
from tests.encoder_set import encoder_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_anchors.txt")


def _golden():
    sec, dec, enc = None, [], []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("["):
            sec = line
            continue
        a, b = line.split()[:2]
        if sec == "[dec]":
            dec.append((int(a, 16), float("nan") if b == "nan" else float.fromhex(b)))
        else:
            enc.append((int(a, 16), int(b, 16)))
    return dec, enc


# ---------------------------------------------------------------- decoder
def test_dec_golden_anchors():
    dec, _ = _golden()
    for code, val in dec:
        got = oracle.dec(np.array([code], np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_dec_all_codes_match_torch():
    got = oracle.dec(np.arange(256, dtype=np.uint8))
    ref = torch_decode_table()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def test_dec_structure():
    v = oracle.dec(np.arange(256, dtype=np.uint8))
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    assert np.array_equal(-v[0x80:0xFF], pos)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.count_nonzero(np.isnan(v)) == 2


# ---------------------------------------------------------------- encoder
def test_enc_golden_anchors():
    _, enc = _golden()
    bits = np.array([b for b, _ in enc], np.uint32)
    want = np.array([c for _, c in enc], np.uint8)
    got = oracle.enc(bits.view(np.float32))
    assert np.array_equal(got, want), [(hex(b), hex(g), hex(w)) for b, g, w in
                                       zip(bits, got, want) if g != w]


def test_enc_exhaustive_roundtrip():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.dec(codes).astype(np.float32)
    back = oracle.enc(vals)
    nan = (codes & 0x7F) == 0x7F
    assert np.array_equal(back[~nan], codes[~nan])
    assert np.all(back[nan] == 0)


def test_enc_encoder_set_vs_bruteforce_and_torch():
    v = encoder_values()
    got = oracle.enc(v)
    assert np.array_equal(got, encode_bruteforce(v))
    inr = np.isfinite(v) & (np.abs(v) <= 464)
    t = torch.from_numpy(v[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inr], t)


@pytest.mark.slow
def test_enc_every_f32_in_the_rounding_range():
    """Every f32 with 2^-11 <= |x| < 2^9, both signs (20 binades x 2^23 x 2),
    against the brute-force nearest-value definition and torch's cast."""
    for e in range(-11, 9):
        base = np.uint32((e + 127) << 23)
        bits = base + np.arange(1 << 23, dtype=np.uint32)
        for sign in (np.uint32(0), np.uint32(0x80000000)):
            x = (bits | sign).view(np.float32)
            got = oracle.enc(x)
            ref = encode_bruteforce(x)
            bad = np.flatnonzero(got != ref)
            assert bad.size == 0, (e, hex(int((bits | sign)[bad[0]])), got[bad[0]], ref[bad[0]])
            if e <= 8:
                inr = np.abs(x) <= 464
                t = torch.from_numpy(x[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                assert np.array_equal(got[inr], t), e


def test_enc_random_bit_patterns():
    g = np.random.Generator(np.random.PCG64(11))
    bits = g.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    assert np.array_equal(oracle.enc(x), encode_bruteforce(x))


# ---------------------------------------------------------------- quantizer
def _rows_for_quantizer():
    g = np.random.Generator(np.random.PCG64(21))
    rows = [g.standard_normal(576).astype(np.float32) for _ in range(64)]
    rows += [(g.standard_normal(576) * 50).astype(np.float32) for _ in range(8)]
    rows += [(g.standard_normal(576) * 1e-30).astype(np.float32) for _ in range(4)]
    rows += [(g.standard_normal(576) * 1e30).astype(np.float32) for _ in range(4)]
    r = g.standard_normal(576).astype(np.float32)
    r[[3, 99]] = np.inf
    r[7] = -np.inf
    r[[11, 500]] = np.nan
    r[13] = -np.nan
    rows.append(r)
    rows.append(np.zeros(576, np.float32))
    z = np.zeros(576, np.float32)
    z[::3] = -0.0
    rows.append(z)
    for amax in (1e-40, 1e-37, np.finfo(np.float32).tiny, 1.30e-36, 1.33e-36, 1.4e-36):
        t = (g.uniform(-1, 1, 576) * amax).astype(np.float32)
        t[5] = np.float32(amax)
        rows.append(t)
    return np.stack(rows)


def test_quantize_rows_against_definition_pieces():
    x = _rows_for_quantizer()
    codes, scales = oracle.quantize_rows(x)
    f32max = np.finfo(np.float32).max
    for i in range(x.shape[0]):
        r = x[i]
        fin = np.isfinite(r)
        amax = np.float32(np.max(np.abs(r[fin]))) if fin.any() else np.float32(0)
        with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
            sc = np.float32(amax) / np.float32(448)
            inv = np.float32(448) / np.float32(amax)
            if not (inv <= f32max):
                inv = np.float32(0)
            y = (r * inv).astype(np.float32)
        assert scales[i].view(np.uint32) == np.float32(sc).view(np.uint32), i
        assert np.array_equal(codes[i], encode_bruteforce(y)), i
        if inv > 0:
            inr = np.isfinite(y)
            t = torch.from_numpy(y[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[i][inr], t), i


def test_quantize_invariants():
    x = _rows_for_quantizer()
    codes, scales = oracle.quantize_rows(x)
    for i in range(x.shape[0]):
        r, c, s = x[i], codes[i], scales[i]
        fin = np.isfinite(r)
        amax = np.float32(np.max(np.abs(r[fin]))) if fin.any() else np.float32(0)
        with np.errstate(divide="ignore", over="ignore"):
            inv = np.float32(448) / amax
        if not np.isfinite(inv):
            # zero row or guarded row: signed zeros (NaN -> +0)
            assert np.all((c & 0x7F) == 0), i
            assert np.array_equal(c == 0x80, np.signbit(r) & ~np.isnan(r)), i
            continue
        # the row's largest finite element lands on +/-448
        k = np.argmax(np.where(fin, np.abs(r), -1))
        assert c[k] & 0x7F == 0x7E
        # NaN -> 0x00, +/-inf -> +/-448
        assert np.all(c[np.isnan(r)] == 0)
        assert np.all(c[np.isposinf(r)] == 0x7E) and np.all(c[np.isneginf(r)] == 0xFE)
        if s >= np.finfo(np.float32).tiny:
            # normal-range scale: every finite element is within half an e4m3
            # gap (times scale) of x, up to the f32 roundings of scale and inv
            deq = oracle.dec(c).astype(np.float64) * float(s)
            err = np.abs(deq[fin] - r[fin].astype(np.float64))
            bound = half_gap(c[fin]) * float(s) * (1 + 2.0 ** -20) + np.abs(
                r[fin].astype(np.float64)) * 2.0 ** -22
            assert np.all(err <= bound), i


def test_quantize_guard_boundary():
    f32max = np.finfo(np.float32).max
    bound = np.float32(448) / f32max  # amax below this makes 448/amax overflow
    for amax in (np.nextafter(bound, np.float32(0)), bound, np.nextafter(bound, np.float32(1))):
        r = np.zeros(576, np.float32)
        r[0] = amax
        r[1] = -amax / 2
        c, s = oracle.quantize_rows(r[None])
        with np.errstate(divide="ignore", over="ignore"):
            inv = np.float32(448) / np.float32(amax)
        if np.isfinite(inv):
            assert c[0, 0] == 0x7E and c[0, 1] == encode_bruteforce(np.float32(-amax / 2 * inv))
        else:
            assert c[0, 0] == 0 and c[0, 1] == 0x80
        assert s[0] == np.float32(amax) / np.float32(448)


# ---------------------------------------------------------------- attention
def _shadow(n, lc=64, rc=16, seed=0, scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    x = (g.standard_normal((n, lc + rc)) * scale).astype(np.float32)
    return oracle.quantize_rows(x)


def _q(h, lc=64, rc=16, seed=1, scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    return ((g.standard_normal((h, lc)) * scale).astype(np.float32),
            (g.standard_normal((h, rc)) * scale).astype(np.float32))


def _deq(codes, scales):
    return oracle.dec(codes) * scales.astype(np.float64)[:, None]


def test_attend_single_row_is_that_row():
    codes, sc = _shadow(1)
    ql, qr = _q(3)
    out, lse = oracle.decode(codes, sc, 1, 64, 16, ql, qr, 0.25)
    k = _deq(codes, sc)[0]
    assert np.array_equal(out, np.broadcast_to(k[:64], out.shape))
    s = float(np.float32(0.25)) * (np.concatenate([ql, qr], 1).astype(np.float64) @ k)
    assert np.allclose(lse, s, rtol=0, atol=1e-12)


def test_attend_identical_rows_and_zero_query():
    codes, sc = _shadow(1, seed=3)
    codes = np.repeat(codes, 37, 0)
    sc = np.repeat(sc, 37)
    ql, qr = _q(2)
    out, lse = oracle.decode(codes, sc, 37, 64, 16, ql, qr, 0.3)
    k = _deq(codes[:1], sc[:1])[0]
    assert np.allclose(out, k[:64], rtol=1e-14, atol=0)
    # q = 0: uniform softmax -> mean of the value parts, lse = ln T
    codes2, sc2 = _shadow(50, seed=4)
    z = np.zeros((2, 64), np.float32), np.zeros((2, 16), np.float32)
    out2, lse2 = oracle.decode(codes2, sc2, 50, 64, 16, z[0], z[1], 0.3)
    assert np.allclose(out2, _deq(codes2, sc2)[:, :64].mean(0), rtol=1e-13, atol=1e-15)
    assert np.allclose(lse2, math.log(50), rtol=0, atol=1e-13)


def test_attend_two_rows_closed_form():
    codes, sc = _shadow(2, seed=5)
    ql, qr = _q(4, seed=6)
    sm = float(np.float32(0.2))  # the oracle takes sm_scale as an f32
    out, lse = oracle.decode(codes, sc, 2, 64, 16, ql, qr, sm)
    k = _deq(codes, sc)
    q = np.concatenate([ql, qr], 1).astype(np.float64)
    s = sm * (q @ k.T)                               # [H, 2]
    gap = s[:, 0] - s[:, 1]
    want = (k[0, :64][None] + np.exp(-gap)[:, None] * k[1, :64][None]) / (1 + np.exp(-gap))[:, None]
    assert np.allclose(out, want, rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, s[:, 0] + np.log1p(np.exp(-gap)), rtol=0, atol=1e-13)


@pytest.mark.parametrize("t", [1, 2, 3, 5, 8])
def test_attend_long_double_brute_force(t):
    codes, sc = _shadow(t, seed=10 + t, scale=3.0)
    ql, qr = _q(3, seed=20 + t, scale=2.0)
    sm = 1 / math.sqrt(80)
    out, lse = oracle.decode(codes, sc, t, 64, 16, ql, qr, sm)
    # textbook softmax in long double, no max subtraction, values from torch's
    # decode table (independent of the oracle's decoder)
    tab = torch_decode_table().astype(np.longdouble)
    k = tab[codes] * sc.astype(np.longdouble)[:, None]
    q = np.concatenate([ql, qr], 1).astype(np.longdouble)
    e = np.exp(np.longdouble(np.float32(sm)) * (q @ k.T))
    want = (e @ k[:, :64]) / e.sum(1, keepdims=True)
    assert np.allclose(out, want.astype(np.float64), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, np.log(e.sum(1)).astype(np.float64), rtol=0, atol=1e-12)


def test_attend_rope_part_matters():
    """q_lat = 0, q_rope != 0: the scores come from the rope columns alone."""
    codes, sc = _shadow(9, seed=30)
    ql, qr = _q(2, seed=31)
    ql[:] = 0
    out, lse = oracle.decode(codes, sc, 9, 64, 16, ql, qr, 0.5)
    k = _deq(codes, sc)
    s = float(np.float32(0.5)) * (qr.astype(np.float64) @ k[:, 64:].T)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(out, p @ k[:, :64], rtol=1e-13, atol=1e-15)


def test_attend_matches_numpy_float64_definition():
    codes, sc = _shadow(300, seed=40, scale=2.0)
    ql, qr = _q(5, seed=41)
    sm = 1 / math.sqrt(80)
    out, lse = oracle.decode(codes, sc, 300, 64, 16, ql, qr, sm)
    k = torch_decode_table()[codes] * sc.astype(np.float64)[:, None]
    s = float(np.float32(sm)) * (np.concatenate([ql, qr], 1).astype(np.float64) @ k.T)
    m = s.max(1, keepdims=True)
    p = np.exp(s - m)
    want = (p @ k[:, :64]) / p.sum(1, keepdims=True)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-15)
    assert np.allclose(lse, (m[:, 0] + np.log(p.sum(1))), rtol=0, atol=1e-12)


def test_attend_permutation_invariance_via_selection():
    codes, sc = _shadow(200, seed=50)
    ql, qr = _q(3, seed=51)
    out, lse = oracle.decode(codes, sc, 200, 64, 16, ql, qr, 0.3)
    perm = np.random.Generator(np.random.PCG64(52)).permutation(200).astype(np.int32)
    o2, l2 = oracle.decode_sel(codes, sc, 200, 64, 16, perm, ql, qr, 0.3)
    assert np.allclose(o2, out, rtol=1e-13, atol=1e-15) and np.allclose(l2, lse, atol=1e-13)


@pytest.mark.parametrize("p", [1, 2, 7, 64, 200])
def test_split_t_merge_equals_dense(p):
    codes, sc = _shadow(200, seed=60, scale=4.0)
    ql, qr = _q(4, seed=61, scale=2.0)
    out, lse = oracle.decode(codes, sc, 200, 64, 16, ql, qr, 0.3)
    o2, l2 = oracle.decode_chunked(codes, sc, 200, 64, 16, ql, qr, 0.3, p)
    assert np.allclose(o2, out, rtol=1e-12, atol=1e-15)
    assert np.allclose(l2, lse, rtol=0, atol=1e-12)


def test_sel_all_rows_single_row_and_out_of_range():
    codes, sc = _shadow(100, seed=70)
    ql, qr = _q(3, seed=71)
    out, lse = oracle.decode(codes, sc, 100, 64, 16, ql, qr, 0.3)
    o, l = oracle.decode_sel(codes, sc, 100, 64, 16, np.arange(100, dtype=np.int32), ql, qr, 0.3)
    assert np.array_equal(o, out) and np.array_equal(l, lse)
    k = _deq(codes, sc)
    o, l = oracle.decode_sel(codes, sc, 100, 64, 16, np.array([17], np.int32), ql, qr, 0.3)
    assert np.array_equal(o, np.broadcast_to(k[17, :64], o.shape))
    sel = np.array([3, 90, 41], np.int32)
    junk = np.array([-1, 100, 3, 90, 1 << 30, 41, -7], np.int32)
    o1, l1 = oracle.decode_sel(codes, sc, 100, 64, 16, sel, ql, qr, 0.3)
    o2, l2 = oracle.decode_sel(codes, sc, 100, 64, 16, junk, ql, qr, 0.3)
    assert np.allclose(o1, o2, rtol=1e-14, atol=0) and np.allclose(l1, l2, atol=1e-14)
    o3, l3 = oracle.decode_sel(codes, sc, 100, 64, 16, np.array([-1, 100], np.int32), ql, qr, 0.3)
    assert np.all(o3 == 0) and np.all(np.isneginf(l3))


def test_sel_multiset_weights():
    codes, sc = _shadow(10, seed=80)
    ql, qr = _q(2, seed=81)
    k = _deq(codes, sc)
    o, l = oracle.decode_sel(codes, sc, 10, 64, 16, np.array([4, 4, 4, 7], np.int32), ql, qr, 0.3)
    s = float(np.float32(0.3)) * (np.concatenate([ql, qr], 1).astype(np.float64) @ k[[4, 7]].T)
    w = np.exp(s - s.max(1, keepdims=True)) * np.array([3.0, 1.0])
    want = (w @ k[[4, 7], :64]) / w.sum(1, keepdims=True)
    assert np.allclose(o, want, rtol=1e-13, atol=1e-15)


def test_batch_rows_are_prefix_decodes():
    codes, sc = _shadow(120, seed=90)
    g = np.random.Generator(np.random.PCG64(91))
    ql = g.standard_normal((6, 3, 64)).astype(np.float32)
    qr = g.standard_normal((6, 3, 16)).astype(np.float32)
    out, lse = oracle.batch(codes, sc, 120, 64, 16, ql, qr, 114, 0.3)
    for s in range(6):
        o, l = oracle.decode(codes, sc, 114 + s + 1, 64, 16, ql[s], qr[s], 0.3)
        assert np.array_equal(out[s], o) and np.array_equal(lse[s], l)
