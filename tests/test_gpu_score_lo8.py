"""GPU parity of the default score path of the e4m3 512/64 decode (fp16 hi +
e4m3 lo query terms, the lo term on the e4m3 MFMA) through the C ABI:

* against the fp64 oracle run with the query that path attends with
  (oracle.query_lo8): scores of f32 grade, so on the x50 outlier caches the
  per-vector worst stays <= 0.5 of the bar, as for the f32_scores path;
* against the exact-query oracle, the contract's bar: the quantized lo term
  adds up to about 0.35 of it on the x50 recipe (30 seeds measured), so the
  same <= 0.5 holds, seeds 1 and 5 (the outlier test's) and 23 included;
* mla8_opts.f32_scores (fp16 hi + lo on the fp16 MFMA) changes the result
  there and nowhere else;
* the packed hardware e4m3 encoder that builds the lo term equals the
  oracle's encoder on that term's whole input domain.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from fp8_mla_latent_amd import workloads as W
from tests.tolerance import check_attention

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_mla_latent_amd import mla8
    return mla8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _outlier_case(seed):
    t, h, lc, rc = 4096, 128, 512, 64
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((t, lc + rc)).astype(np.float32)
    idx = g.choice(t, int(round(0.01 * t)), replace=False)
    x[idx] *= np.float32(50.0)
    q = g.standard_normal((h, lc + rc)).astype(np.float32)
    return x, np.ascontiguousarray(q[:, :lc]), np.ascontiguousarray(q[:, lc:])


@pytest.mark.parametrize("seed", [1, 5, 23])
def test_lo8_decode_matches_its_query_reading(m, seed):
    lc, rc, sm = 512, 64, 1.0 / math.sqrt(192.0)
    say(f"e4m3-lo score decode, x50 outlier recipe seed {seed}")
    x, ql, qr = _outlier_case(seed)
    t = x.shape[0]
    codes, scales = m.mla8_quantize_rows(dev(x), lc, rc)
    out8, lse8 = m.mla8_decode(codes, scales, t, lc, rc, dev(ql), dev(qr), sm)
    out, _ = m.mla8_decode(codes, scales, t, lc, rc, dev(ql), dev(qr), sm, f32_scores=True)
    oc, os_ = host(codes), host(scales)
    qql, qqr = oracle.query_lo8(ql, qr, sm)
    r8, l8 = oracle.decode(oc, os_, t, lc, rc, qql, qqr, sm)
    worst = check_attention(host(out8), r8, host(lse8), l8, f"e4m3-lo reading seed {seed}",
                            outliers=True)
    say(f"  worst err/bar against the quantized-query oracle {worst:.4f}")
    assert worst <= 0.5
    ro, rl = oracle.decode(oc, os_, t, lc, rc, ql, qr, sm)
    worst_exact = check_attention(host(out8), ro, host(lse8), rl, f"e4m3-lo exact seed {seed}",
                                  outliers=True)
    say(f"  worst err/bar against the exact-query oracle {worst_exact:.4f}")
    assert worst_exact <= 0.5
    # the option takes effect: f32_scores attends with the f32 query
    assert not np.array_equal(host(out8), host(out))


@pytest.mark.parametrize("h,t,splits", [(40, 700, 0), (16, 300, 3), (8, 64, 1)])
def test_lo8_partial_head_group(m, h, t, splits):
    """Head counts that leave the last group of 32 partly empty: the path's
    result per head equals the oracle with that head's query_lo8 reading, and
    the outputs of the heads past H are never written."""
    lc, rc, sm = 512, 64, 1.0 / math.sqrt(192.0)
    say(f"e4m3-lo decode, H={h} T={t} splits={splits}")
    g = np.random.Generator(np.random.PCG64(700 + h + t))
    x = (g.standard_normal((t, lc + rc)) * g.uniform(0.5, 2, (t, 1))).astype(np.float32)
    ql = g.standard_normal((h, lc)).astype(np.float32)
    qr = g.standard_normal((h, rc)).astype(np.float32)
    codes, scales = m.mla8_quantize_rows(dev(x), lc, rc)
    if splits == 0:
        splits = m.mla8_plan_splits(m.MLA8_OP_DECODE, t, h)
    out8, lse8 = m.mla8_decode(codes, scales, t, lc, rc, dev(ql), dev(qr), sm, n_splits=splits)
    qql, qqr = oracle.query_lo8(ql, qr, sm)
    r8, l8 = oracle.decode(host(codes), host(scales), t, lc, rc, qql, qqr, sm)
    check_attention(host(out8), r8, host(lse8), l8, f"H={h} T={t}", few_rows=True)
    # the same heads as the leading H of a full group give the same result
    hf = 32 * ((h + 31) // 32)
    qlf = np.concatenate([ql, np.repeat(ql[-1:], hf - h, 0)])
    qrf = np.concatenate([qr, np.repeat(qr[-1:], hf - h, 0)])
    outf, lsef = m.mla8_decode(codes, scales, t, lc, rc, dev(qlf), dev(qrf), sm, n_splits=splits)
    np.testing.assert_array_equal(host(outf)[:h], host(out8))
    np.testing.assert_array_equal(host(lsef)[:h], host(lse8))


def test_lo8_fused_step_full_size(m):
    """The long-context step (262143 rows + one fresh row, 64 heads, 128
    chunks) on the default e4m3-lo scores: fused append + decode bit for bit
    equal to append then decode, and every head against the quantized-query
    oracle (the exact-query comparison is test_long_context_step_full)."""
    w = W.LONG
    T = w.t_rows
    say(f"{w.name}: e4m3-lo score fused step")
    x = W.rows(w, T)
    shadows = []
    for _ in range(2):
        codes = torch.zeros((T, w.d), dtype=torch.uint8, device=DEV)
        scales = torch.zeros((T,), dtype=torch.float32, device=DEV)
        assert m.mla8_append(codes, scales, 0, dev(x[:-1]), w.lc, w.rc) == T - 1
        shadows.append((codes, scales))
    ql, qr = W.queries(w)
    (ca, sa), (cb, sb) = shadows
    ob, lb, tb = m.mla8_append_decode(cb, sb, T - 1, dev(x[-1:]), w.lc, w.rc, dev(ql), dev(qr),
                                      w.sm_scale)
    assert tb == T
    assert m.mla8_append(ca, sa, T - 1, dev(x[-1:]), w.lc, w.rc) == T
    oa, la = m.mla8_decode(ca, sa, T, w.lc, w.rc, dev(ql), dev(qr), w.sm_scale)
    assert np.array_equal(host(oa), host(ob)) and np.array_equal(host(la), host(lb))
    qql, qqr = oracle.query_lo8(ql, qr, w.sm_scale)
    ro, rl = oracle.decode(host(cb), host(sb), T, w.lc, w.rc, qql, qqr, w.sm_scale)
    worst = check_attention(host(ob), ro, host(lb), rl, f"{w.name} e4m3-lo reading")
    say(f"  worst elementwise err/bar {worst:.4f}")


def test_lo8_noalloc_matches_workspace_call(m):
    w = W.DSV3
    t_old, n_new = 3000, 2
    say("e4m3-lo scores: static-scratch step against the workspace step")
    x = W.rows(w, t_old + n_new, seed_offset=7)
    ql, qr = W.queries(w, seed_offset=7)
    res = []
    for noalloc in (False, True):
        codes = torch.zeros((t_old + n_new, w.d), dtype=torch.uint8, device=DEV)
        scales = torch.zeros((t_old + n_new,), dtype=torch.float32, device=DEV)
        assert m.mla8_append(codes, scales, 0, dev(x[:t_old]), w.lc, w.rc) == t_old
        if noalloc:
            out = torch.empty((w.n_heads, w.lc), dtype=torch.float32, device=DEV)
            lse = torch.empty((w.n_heads,), dtype=torch.float32, device=DEV)
            assert m.mla8_append_decode_noalloc(codes, scales, t_old, dev(x[t_old:]), w.lc, w.rc,
                                                dev(ql), dev(qr), w.sm_scale, out,
                                                lse) == t_old + n_new
        else:
            out, lse, _ = m.mla8_append_decode(codes, scales, t_old, dev(x[t_old:]), w.lc, w.rc,
                                               dev(ql), dev(qr), w.sm_scale)
        res.append((host(out), host(lse)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def test_f32_scores_ignored_outside_the_e4m3_lo_shape(m):
    # tiny rows (lc = 64, rc = 16) take the general kernel: the option changes nothing
    w = W.TINY
    say("f32_scores on a shape without the e4m3-lo score path")
    x = W.rows(w, w.t_rows)
    ql, qr = W.queries(w)
    codes, scales = m.mla8_quantize_rows(dev(x), w.lc, w.rc)
    a = m.mla8_decode(codes, scales, w.t_rows, w.lc, w.rc, dev(ql), dev(qr), w.sm_scale)
    b = m.mla8_decode(codes, scales, w.t_rows, w.lc, w.rc, dev(ql), dev(qr), w.sm_scale,
                      f32_scores=True)
    assert np.array_equal(host(a[0]), host(b[0])) and np.array_equal(host(a[1]), host(b[1]))


@pytest.mark.parametrize("h,n_q,pos0,splits", [(32, 80, 63, 3), (64, 6, 700, 5), (96, 2, 130, 0),
                                               (64, 3, 4000, 0)], ids=lambda v: str(v))
def test_lo8_causal_batch(m, h, n_q, pos0, splits):
    """The causal batch on the e4m3-lo score path (e4m3 rows, 512/64, n_heads
    a multiple of 32, pos0 >= 63): chunks that end before a query's position
    (empty partials), ragged last tiles whose leading rows belong to the
    previous tile, several head groups per query.  The default call against
    the quantized-query oracle and against the exact query; f32_scores against
    the exact query."""
    lc, rc, sm = 512, 64, 1.0 / math.sqrt(192.0)
    t = pos0 + n_q
    say(f"e4m3-lo causal batch H={h} S={n_q} pos0={pos0} splits={splits}")
    g = np.random.Generator(np.random.PCG64(h * 1000 + n_q))
    x = g.standard_normal((t, lc + rc)).astype(np.float32)
    ql = g.standard_normal((n_q, h, lc)).astype(np.float32)
    qr = g.standard_normal((n_q, h, rc)).astype(np.float32)
    codes, scales = m.mla8_quantize_rows(dev(x), lc, rc)
    oc, os_ = host(codes), host(scales)
    # prefixes of a few hundred rows: the per-vector form (short causal prefix)
    few = pos0 < 2000
    out8, lse8 = m.mla8_batch(codes, scales, t, lc, rc, dev(ql), dev(qr), pos0, sm,
                              n_splits=splits)
    qql, qqr = oracle.query_lo8(ql.reshape(-1, lc), qr.reshape(-1, rc), sm)
    r8, l8 = oracle.batch(oc, os_, t, lc, rc, qql.reshape(n_q, h, lc), qqr.reshape(n_q, h, rc),
                          pos0, sm)
    w8 = check_attention(host(out8), r8, host(lse8), l8, "e4m3-lo batch, its reading",
                         few_rows=few)
    ro, rl = oracle.batch(oc, os_, t, lc, rc, ql, qr, pos0, sm)
    we = check_attention(host(out8), ro, host(lse8), rl, "e4m3-lo batch, exact query",
                         few_rows=few)
    out, lse = m.mla8_batch(codes, scales, t, lc, rc, dev(ql), dev(qr), pos0, sm,
                            n_splits=splits, f32_scores=True)
    wf = check_attention(host(out), ro, host(lse), rl, "f32_scores batch, exact query",
                         few_rows=few)
    say(f"  worst err/bar: reading {w8:.4f}, exact {we:.4f}, f32_scores {wf:.4f}")


def test_lo_term_encoder_matches_the_oracle(m):
    """The packed hardware e4m3 encoder of the lo term (mla8_test_encode_pk)
    against oracle.enc on every input the decode can give it: the lo term is
    an fp16 value scaled by 2^j to below 256, so every finite fp16 value times
    2^j, j in [-40, 40], with |y| < 448 (5 M values, both signs, the e4m3
    subnormal and underflow ranges and every rounding tie included)."""
    say("packed e4m3 encoder of the lo term against the oracle")
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h)]
    parts = []
    for j in range(-40, 41):
        y = np.ldexp(h, j).astype(np.float32)
        parts.append(y[np.isfinite(y) & (np.abs(y) < 448.0)])
    x = np.concatenate(parts)
    x = np.concatenate([x, np.zeros((-x.size) % 4, np.float32)])
    got = host(m.mla8_test_encode_pk(dev(x)))
    ref = oracle.enc(x)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (int(bad.size), float(x[bad[0]]), int(got[bad[0]]), int(ref[bad[0]]))


def test_f32_scores_switches_the_mixed_path(m):
    """On mixed rows (448/64) the option selects the other kernel: the default
    attends with query_lo8_mx's query, f32_scores with the query as given, so
    the two results differ (and each matches its own reference elsewhere)."""
    lc, rc, sm = 448, 64, 1.0 / math.sqrt(192.0)
    t, h = 3000, 64
    say("f32_scores on mixed rows")
    g = np.random.Generator(np.random.PCG64(71))
    x = g.standard_normal((t, lc + rc)).astype(np.float32)
    ql = g.standard_normal((h, lc)).astype(np.float32)
    qr = g.standard_normal((h, rc)).astype(np.float32)
    rows, sc = m.mla8_quantize_rows_mx(dev(x), lc, rc)
    a, _ = m.mla8_decode_mx(rows, sc, t, lc, rc, dev(ql), dev(qr), sm)
    b, _ = m.mla8_decode_mx(rows, sc, t, lc, rc, dev(ql), dev(qr), sm, f32_scores=True)
    assert not np.array_equal(host(a), host(b))


@pytest.mark.parametrize("mode", ["sel", "batch", "sel_mx"])
def test_graph_replays_of_the_gather_and_batch_paths(m, mode):
    """The gathered, causal and mixed gathered calls on the 32x32 kernel
    captured once and replayed, with eager work between replays: every replay
    equals the eager result bit for bit."""
    say(f"graph replay: {mode}")
    g = np.random.Generator(np.random.PCG64(81))
    sm = 1.0 / math.sqrt(192.0)
    if mode == "sel_mx":
        lc, rc, t, h = 448, 64, 6000, 64
        x = g.standard_normal((t, lc + rc)).astype(np.float32)
        codes, sc = m.mla8_quantize_rows_mx(dev(x), lc, rc)
    else:
        lc, rc, t, h = 512, 64, 6000, 64
        x = g.standard_normal((t, lc + rc)).astype(np.float32)
        codes, sc = m.mla8_quantize_rows(dev(x), lc, rc)
    sel = dev(np.sort(g.choice(t, 700, replace=False)).astype(np.int32))
    n_q = 4
    if mode == "batch":
        ql = dev(g.standard_normal((n_q, h, lc)).astype(np.float32))
        qr = dev(g.standard_normal((n_q, h, rc)).astype(np.float32))
        out = torch.empty((n_q, h, lc), dtype=torch.float32, device=DEV)
        lse = torch.empty((n_q, h), dtype=torch.float32, device=DEV)
        ws = torch.empty(m.mla8_workspace_bytes(m.MLA8_OP_BATCH, t, h, n_q, lc), dtype=torch.uint8,
                         device=DEV)
    else:
        ql = dev(g.standard_normal((h, lc)).astype(np.float32))
        qr = dev(g.standard_normal((h, rc)).astype(np.float32))
        out = torch.empty((h, lc), dtype=torch.float32, device=DEV)
        lse = torch.empty((h,), dtype=torch.float32, device=DEV)
        ws = torch.empty(m.mla8_workspace_bytes(m.MLA8_OP_DECODE_SEL, 700, h, 1, lc),
                         dtype=torch.uint8, device=DEV)

    def call():
        if mode == "sel":
            m.mla8_decode_sel(codes, sc, t, lc, rc, sel, ql, qr, sm, out=out, lse=lse, workspace=ws)
        elif mode == "sel_mx":
            m.mla8_decode_sel_mx(codes, sc, t, lc, rc, sel, ql, qr, sm, out=out, lse=lse,
                                 workspace=ws)
        else:
            m.mla8_batch(codes, sc, t, lc, rc, ql, qr, t - n_q, sm, out=out, lse=lse, workspace=ws)

    call()
    ref_out, ref_lse = host(out).copy(), host(lse).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call()
    for r in range(4):
        out.zero_()
        lse.zero_()
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref_out), r
        assert np.array_equal(host(lse), ref_lse), r
        _ = (torch.ones(1000, device=DEV) * 2).sum().item()  # eager work between replays
