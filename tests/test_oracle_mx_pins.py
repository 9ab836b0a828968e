"""Pins for the oracle's mixed row layout (no GPU).

Page passage: "B1 Mixed FP8/BF16 FMHA first pass", the storage-format list:
noPE KV as e4m3 bytes with a per-row f32 scale, RoPE KV kept in bf16, in the
512 / 448 / 64 shape.  The bf16 encoder is pinned to torch's float32 ->
bfloat16 cast (round to nearest even) and its decoder to torch's bfloat16 ->
float; the mixed quantizer to the (separately pinned) row quantizer on the noPE
part plus the bf16 encoder on the RoPE part; the mixed decode to a float64
numpy softmax attention on inputs that the format represents exactly, with
per-row power-of-two noPE scales that must not touch the RoPE part.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle


def torch_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_random_bit_patterns_match_torch():
    g = np.random.Generator(np.random.PCG64(41))
    bits = g.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    np.testing.assert_array_equal(oracle.bf16(x), torch_bf16_bits(x))


def test_bf16_ties_subnormals_and_edges():
    vals = []
    for e in range(-133, 128):
        for m in (0, 1, 2, 3, 0x7E, 0x7F):
            base = np.float32(np.ldexp(1.0 + m / 128.0, e)) if e >= -126 else \
                np.float32(np.ldexp(m, e))
            b = base.view(np.uint32)
            for d in (0, 0x7FFF, 0x8000, 0x8001, 0xFFFF):  # below, at and above the tie
                vals.append(np.uint32(int(b) + d if int(b) + d < 2 ** 32 else int(b)))
    x = np.array(vals, np.uint32).view(np.float32)
    x = np.concatenate([x, -x, np.array([np.finfo(np.float32).max, np.inf, -np.inf, 0.0, -0.0],
                                        np.float32)])
    x = x[~np.isnan(x)]
    np.testing.assert_array_equal(oracle.bf16(x), torch_bf16_bits(x))
    assert oracle.bf16(np.float32(np.finfo(np.float32).max)) == 0x7F80  # rounds to inf
    assert oracle.bf16(np.float32(np.nan)) == 0x7FC0
    assert oracle.bf16(-np.float32(np.nan)) == 0xFFC0


def test_bf16_value_all_patterns_match_torch():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_value(b)
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])


def test_quantize_rows_mx_is_row_quantizer_plus_bf16():
    g = np.random.Generator(np.random.PCG64(42))
    lc, rc = 448, 64
    x = g.standard_normal((50, lc + rc)).astype(np.float32)
    x[3, 10] = np.nan
    x[7, lc + 5] = np.inf
    x[9, :lc] *= 1e-38  # guard row on the noPE part
    rows, sc = oracle.quantize_rows_mx(x, lc, rc)
    c_ref, s_ref = oracle.quantize_rows(x[:, :lc])
    np.testing.assert_array_equal(rows[:, :lc], c_ref)
    np.testing.assert_array_equal(sc.view(np.uint32), s_ref.view(np.uint32))
    rope = rows[:, lc:].copy().view(np.uint16)  # little-endian pairs
    np.testing.assert_array_equal(rope, oracle.bf16(x[:, lc:]))


E4M3_EXACT = np.array([0.0, 0.5, 0.75, 1.0, 1.5, 2.0, 3.0, 5.0, 6.0, 10.0, 14.0, 24.0, 40.0],
                      np.float32)


def _attention(k, v, q, sm):
    s = sm * (k @ q)
    p = np.exp(s - s.max())
    return (p @ v) / p.sum(), s.max() + np.log(p.sum())


@pytest.mark.parametrize("lc,rc", [(448, 64), (64, 32)])
def test_decode_mx_closed_form_with_noPE_only_scales(lc, rc):
    g = np.random.Generator(np.random.PCG64(43 + lc))
    t, h = 37, 3
    nope = g.choice(E4M3_EXACT, (t, lc)) * g.choice([-1.0, 1.0], (t, lc))
    nope[np.arange(t), g.integers(0, lc, t)] = 448.0
    a = g.integers(-8, 6, t)
    nope = nope * np.exp2(a)[:, None]          # row scale exactly 2^a_t
    rope = np.round(g.standard_normal((t, rc)) * 8) / 8  # bf16-exact, unscaled
    x = np.concatenate([nope, rope], axis=1).astype(np.float32)
    rows, sc = oracle.quantize_rows_mx(x, lc, rc)
    np.testing.assert_array_equal(sc, np.exp2(a).astype(np.float32))
    ql = g.standard_normal((h, lc)).astype(np.float32) * 0.02
    qr = g.standard_normal((h, rc)).astype(np.float32) * 0.3
    sm = float(np.float32(1.0 / np.sqrt(192.0)))  # the API takes sm_scale as f32
    out, lse = oracle.decode_mx(rows, sc, t, lc, rc, ql, qr, sm)
    k = x.astype(np.float64)
    for i in range(h):
        q = np.concatenate([ql[i], qr[i]]).astype(np.float64)
        o, l = _attention(k, k[:, :lc], q, sm)
        np.testing.assert_allclose(out[i], o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[i], l, rtol=1e-12)


def test_decode_sel_mx_identities():
    # the selection of every row is the dense decode; a repeated row counts as
    # often as it appears (closed form: weight 2 for a doubled row);
    # out-of-range entries are skipped
    g = np.random.Generator(np.random.PCG64(44))
    lc, rc, t, h = 448, 64, 50, 4
    x = g.standard_normal((t, lc + rc)).astype(np.float32)
    rows, sc = oracle.quantize_rows_mx(x, lc, rc)
    ql = g.standard_normal((h, lc)).astype(np.float32)
    qr = g.standard_normal((h, rc)).astype(np.float32)
    sm = 0.07
    d_out, d_lse = oracle.decode_mx(rows, sc, t, lc, rc, ql, qr, sm)
    s_out, s_lse = oracle.decode_sel_mx(rows, sc, t, lc, rc, np.arange(t)[::-1], ql, qr, sm)
    np.testing.assert_allclose(s_out, d_out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s_lse, d_lse, rtol=1e-12)
    o1, l1 = oracle.decode_sel_mx(rows, sc, t, lc, rc, np.array([7, -1, 9, 7, t + 3]), ql, qr, sm)
    o2, l2 = oracle.decode_sel_mx(rows, sc, t, lc, rc, np.array([9, 7]), ql, qr, sm)
    # doubled row 7: lse grows by ln(1 + p7) where p7 is row 7's share
    k = oracle.bf16_value(rows[:, lc:].copy().view(np.uint16))
    kn = oracle.dec(rows[:, :lc]) * sc[:, None].astype(np.float64)
    for i in range(h):
        q = np.concatenate([ql[i], qr[i]]).astype(np.float64)
        s7 = np.float32(sm) * (np.concatenate([kn[7], k[7]]) @ q)
        s9 = np.float32(sm) * (np.concatenate([kn[9], k[9]]) @ q)
        mmax = max(s7, s9)
        w7, w9 = 2 * np.exp(s7 - mmax), np.exp(s9 - mmax)
        np.testing.assert_allclose(o1[i], (w7 * kn[7] + w9 * kn[9]) / (w7 + w9), rtol=1e-10,
                                   atol=1e-12)
        np.testing.assert_allclose(l1[i], mmax + np.log(w7 + w9), rtol=1e-12)
    assert not np.allclose(o1, o2)
