"""Pins of oracle.query_lo8, the query that the e4m3 512/64 decode attends with
by default (fp16 hi term plus an e4m3 lo term with a per-head power-of-2
scale; mla8_opts.f32_scores turns it off).  No GPU.

* identity: a query that the fp16 hi term already holds exactly (integers
  times a power-of-2 query scale) has lo = 0, so the reconstructed query is
  the query itself, bit for bit;
* bound: the reconstruction differs from q by at most what the e4m3 rounding
  of lo can leave, 2^-15 of the head's largest |q| (about 2^-16.4 measured);
  a dropped lo term (2^-12), a dropped hi term or a wrong scale exponent
  breaks it, and a reconstruction equal to the fp16 hi term alone would too;
* the e4m3 step against torch's float8_e4m3fn cast on the same scaled values
  (round to nearest even; the values stay below 448, so the saturating and
  the non-saturating encoder agree).

oracle.query_lo8_mx, the mixed-row variant: the same identity and bounds for
the noPE part, whose scaling exponent must ignore the RoPE part (checked with
RoPE values 1e6 times larger), and the RoPE part as two bf16 terms, checked
against torch's bf16 rounding.
"""
import numpy as np
import pytest
import torch

import oracle


def _es_one_scale():
    """An f32 softmax scale whose f32 product with f32(log2 e) is exactly 1."""
    l2e = np.float32(1.4426950408889634)
    s = np.float32(1.0) / l2e
    for _ in range(64):
        p = np.float32(s * l2e)
        if p == np.float32(1.0):
            return float(s)
        s = np.nextafter(s, np.float32(np.inf) if p < 1 else np.float32(0), dtype=np.float32)
    pytest.skip("no f32 scale with an exact unit product found")


def test_fp16_exact_query_reconstructs_exactly():
    sm = _es_one_scale()
    g = np.random.default_rng(3)
    ql = g.integers(-7, 8, size=(5, 512)).astype(np.float32)
    qr = g.integers(-7, 8, size=(5, 64)).astype(np.float32)
    ql[0, 0] = 7.0   # a nonzero head
    a, b = oracle.query_lo8(ql, qr, sm)
    assert np.array_equal(a, ql) and np.array_equal(b, qr)


@pytest.mark.parametrize("scale", [1.0, 50.0, 1e-3])
def test_reconstruction_within_the_lo_rounding_bound(scale):
    sm = 1.0 / np.sqrt(192.0)
    g = np.random.default_rng(11)
    ql = (g.standard_normal((16, 512)) * scale).astype(np.float32)
    qr = (g.standard_normal((16, 64)) * scale).astype(np.float32)
    ql[3, :] *= 50.0   # one head much larger than the others
    a, b = oracle.query_lo8(ql, qr, sm)
    q = np.concatenate([ql, qr], 1).astype(np.float64)
    qq = np.concatenate([a, b], 1).astype(np.float64)
    dev = np.abs(qq - q).max(1) / np.abs(q).max(1)
    assert np.all(dev <= 2.0 ** -15), dev.max()
    # the lo term is there: the fp16 hi term alone misses by about 2^-12
    es = np.float32(np.float32(sm) * np.float32(1.4426950408889634))
    hi_only = []
    for h in range(q.shape[0]):
        e = q[h].astype(np.float32)
        k = 15 - int(np.frexp(np.float32(np.abs(e).max() * es))[1])
        r = (e * np.float32(np.ldexp(es, k))).astype(np.float32)
        hi = r.astype(np.float16).astype(np.float64)
        hi_only.append(np.abs(np.ldexp(hi, -k) / np.float64(es) - q[h]).max() / np.abs(q[h]).max())
    assert np.all(dev < np.array(hi_only) / 8), (dev, hi_only)


def test_e4m3_step_matches_torch():
    g = np.random.default_rng(5)
    v = (g.standard_normal(4096) * 60.0).astype(np.float32)
    v = np.clip(v, -255.0, 255.0).astype(np.float32)
    v[:8] = [0.0, -0.0, 2.0 ** -10, -(2.0 ** -9), 0.001953125 * 3, 255.0, -240.0, 17.5]
    ours = oracle.dec(oracle.enc(v))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# ---- oracle.query_lo8_mx: the mixed-row variant (noPE lo term in e4m3, k over
# the noPE part alone; RoPE as two bf16 terms)

def test_mx_exact_query_reconstructs_exactly():
    """Integer noPE queries with es = 1 are held by the fp16 hi term (lo = 0);
    small-integer RoPE values are bf16 values (their lo term is 0)."""
    sm = _es_one_scale()
    g = np.random.default_rng(13)
    ql = g.integers(-7, 8, size=(4, 448)).astype(np.float32)
    qr = g.integers(-100, 101, size=(4, 64)).astype(np.float32)
    ql[:, 0] = 7.0
    a, b = oracle.query_lo8_mx(ql, qr, sm)
    assert np.array_equal(a, ql) and np.array_equal(b, qr)


@pytest.mark.parametrize("rope_scale", [1.0, 1e6, 1e-6])
def test_mx_bounds_and_noPE_scaling_ignores_rope(rope_scale):
    """noPE within 2^-15 of each head's largest |q_lat| whatever the RoPE
    magnitudes (a k taken over the RoPE part too would leave the noPE part
    with fewer bits when RoPE is 1e6 times larger); RoPE within 2^-16 of each
    element (two bf16 terms hold about 16 bits); and the noPE lo term is there
    (the fp16 hi term alone misses by about 2^-12)."""
    sm = 1.0 / np.sqrt(192.0)
    g = np.random.default_rng(17)
    ql = g.standard_normal((8, 448)).astype(np.float32)
    qr = (g.standard_normal((8, 64)) * rope_scale).astype(np.float32)
    a, b = oracle.query_lo8_mx(ql, qr, sm)
    dev = np.abs(a.astype(np.float64) - ql).max(1) / np.abs(ql).max(1)
    assert np.all(dev <= 2.0 ** -15), dev.max()
    assert np.all(np.abs(b.astype(np.float64) - qr) <= 2.0 ** -16 * np.abs(qr)), \
        float((np.abs(b.astype(np.float64) - qr) / np.abs(qr)).max())
    es = np.float32(np.float32(sm) * np.float32(1.4426950408889634))
    for h in range(ql.shape[0]):
        e = ql[h]
        k = 15 - int(np.frexp(np.float32(np.abs(e).max() * es))[1])
        r = (e * np.float32(np.ldexp(es, k))).astype(np.float32)
        hi = r.astype(np.float16).astype(np.float64)
        hi_dev = np.abs(np.ldexp(hi, -k) / np.float64(es) - ql[h]).max() / np.abs(ql[h]).max()
        assert dev[h] < hi_dev / 8, (h, dev[h], hi_dev)


def test_mx_rope_terms_are_bf16_values():
    """The RoPE reconstruction is the sum of two bf16 values (times 1/es): with
    es = 1 it is exactly bf16(e) + bf16(e - bf16(e)), checked against torch's
    bf16 rounding."""
    sm = _es_one_scale()
    g = np.random.default_rng(19)
    qr = g.standard_normal((3, 64)).astype(np.float32)
    ql = np.ones((3, 448), np.float32)
    _, b = oracle.query_lo8_mx(ql, qr, sm)
    t = torch.from_numpy(qr)
    hi = t.to(torch.bfloat16).to(torch.float32)
    lo = (t - hi).to(torch.bfloat16).to(torch.float32)
    ref = (hi.double() + lo.double()).float().numpy()
    assert np.array_equal(b, ref)
