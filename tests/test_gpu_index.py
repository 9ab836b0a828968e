"""GPU parity of the fp8 indexer score + top-k (mla8_index_topk) against the
fp64 CPU oracle, through the C ABI.

Keys are quantized on the GPU (bit-identical to the oracle's quantizer, checked
here as well).  Scores are compared element by element within a bound derived
from the f32 arithmetic (below).  The selection is checked two ways: exactly,
as the top-k of the GPU's own f32 scores under the selection rule (ties to the
smaller row, NaN lowest, -0 = +0, ascending output); and against the oracle's
fp64 scores, where a chosen row may only be outranked by an unchosen one
within the score bound (near-ties may legitimately resolve either way).

Score bound.  The scaled fp8 MFMA adds its 128 products in aligned groups of
8, each product cut toward zero at 2^(E-13), E the group's largest operand
exponent sum, so a group loses less than 8 * 2^-13 of its largest product;
three f32 products and a sum over at most 64 heads follow.  With A_t = sum_j
|w_j| q_scale_j k_scale_t sum_d |q8_jd k8_td| that gives the contract bound
|I_gpu - I_ref| <= (2^-10 + 2^-16) A_t.  On inputs whose products are of
similar size within a group (random keys and queries, the workload recipe) the
truncations are far smaller: those tests assert 2e-5 A_t, a regression check
of that typical behaviour; test_index_truncation_adversarial builds groups of
one large and seven sub-unit products and asserts the contract bound.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from fp8_mla_latent_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL = 2e-5                      # typical: random-like products
REL_CONTRACT = 2.0 ** -10 + 2.0 ** -16


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


def _bound(kc, ks, q, w, rel=REL):
    qc, qs = oracle.quantize_rows(q)
    aq = np.abs(oracle.dequant(qc, qs))          # [n_ih, 128]
    ak = np.abs(oracle.dequant(kc, ks))          # [T, 128]
    return rel * ((ak @ aq.T) @ np.abs(w.astype(np.float64))) + 1e-30


def _check(sel, s_gpu, s_ref, bound, k, what):
    t = s_ref.size
    kk = min(k, t)
    assert sel.shape == (kk,), what
    assert (np.diff(sel) > 0).all() and sel.min() >= 0 and sel.max() < t, what
    err = np.abs(s_gpu.astype(np.float64) - s_ref)
    fin = np.isfinite(s_ref)
    assert (err[fin] <= bound[fin]).all(), (what, float((err / bound)[fin].max()))
    # exact: the top-k of the GPU's own scores
    np.testing.assert_array_equal(sel, oracle.index_topk(s_gpu.astype(np.float64), k),
                                  err_msg=what)
    # against the oracle: no unchosen row beats a chosen one beyond the bound
    if kk < t:
        chosen = np.zeros(t, bool)
        chosen[sel] = True
        lo = (s_ref + bound)[chosen].min()
        hi = (s_ref - bound)[~chosen].max()
        assert lo >= hi, (what, lo, hi)
    diff = np.setdiff1d(oracle.index_topk(s_ref, k), sel).size
    say(f"  {what}: max err/bound {float((err / bound)[fin].max()):.3f}, "
        f"rows differing from the fp64 selection: {diff}")


def _run(m, keys, q, w, k):
    kd = dev(keys)
    kc, ks = m.mla8_quantize_rows(kd, keys.shape[1], 0)
    qd, wd = dev(q), dev(w)
    sel, sc = m.mla8_index_topk(kc, ks, qd, wd, k, want_scores=True)
    return host(kc), host(ks), host(sel), host(sc)


@pytest.mark.parametrize("t,n_ih,k", [(1, 16, 1), (15, 16, 4), (100, 32, 7), (513, 64, 64),
                                      (5000, 48, 2048), (4096, 64, 4096), (20000, 64, 1)])
def test_index_small(m, t, n_ih, k):
    say(f"index t={t} n_ih={n_ih} k={k}")
    g = np.random.Generator(np.random.PCG64(1000 + t + n_ih + k))
    keys = g.standard_normal((t, 128)).astype(np.float32)
    q = g.standard_normal((n_ih, 128)).astype(np.float32)
    wt = (g.standard_normal(n_ih) / np.sqrt(n_ih)).astype(np.float32)
    kc, ks, sel, sc = _run(m, keys, q, wt, k)
    oc, os_ = oracle.quantize_rows(keys)
    np.testing.assert_array_equal(kc, oc)
    np.testing.assert_array_equal(ks.view(np.uint32), os_.view(np.uint32))
    ref = oracle.index_scores(kc, ks, q, wt)
    _check(sel, sc, ref, _bound(kc, ks, q, wt), k, f"t={t} n_ih={n_ih} k={k}")


def test_index_workload(m):
    w = W.DSA_INDEX
    say(f"index workload {w.name}")
    keys = W.rows(w, w.t_rows)
    q = W.queries(w)[0]
    wt = W.index_weights(w)
    kc, ks, sel, sc = _run(m, keys, q, wt, w.n_sel)
    ref = oracle.index_scores(kc, ks, q, wt)
    _check(sel, sc, ref, _bound(kc, ks, q, wt), w.n_sel, w.name)


def test_index_ties_zero_and_nan_weights(m):
    say("index ties: zero and NaN weights")
    g = np.random.Generator(np.random.PCG64(31))
    keys = g.standard_normal((3000, 128)).astype(np.float32)
    q = g.standard_normal((64, 128)).astype(np.float32)
    for wt, what in [(np.zeros(64, np.float32), "zero"),
                     (np.full(64, np.nan, np.float32), "nan"),
                     (-np.abs(g.standard_normal(64)).astype(np.float32), "nonpositive")]:
        kc, ks, sel, sc = _run(m, keys, q, wt, 500)
        if what != "nonpositive":
            # every score equal (0) or NaN: the first rows win
            np.testing.assert_array_equal(sel, np.arange(500, dtype=np.int32), err_msg=what)
        ref = oracle.index_scores(kc, ks, q, wt)
        np.testing.assert_array_equal(sel, oracle.index_topk(sc.astype(np.float64), 500),
                                      err_msg=what)
        if what == "zero":
            assert (sc == 0).all()


def test_index_many_equal_scores_take_the_global_path(m):
    # 20000 equal scores: more candidates than the LDS holds, so the last
    # workgroup selects in global memory; the first rows win
    say("index: 20000 tied candidates")
    g = np.random.Generator(np.random.PCG64(34))
    keys = g.standard_normal((20000, 128)).astype(np.float32)
    q = g.standard_normal((32, 128)).astype(np.float32)
    kc, ks, sel, sc = _run(m, keys, q, np.zeros(32, np.float32), 3000)
    np.testing.assert_array_equal(sel, np.arange(3000, dtype=np.int32))
    # half the rows tied at the top: the tie cut still goes by row index
    wt = np.abs(g.standard_normal(32)).astype(np.float32)
    keys2 = keys.copy()
    top = np.sort(g.choice(20000, 15000, replace=False))
    qs = q.astype(np.float64).sum(axis=0)
    keys2[top] = (30.0 * qs / np.linalg.norm(qs)).astype(np.float32)  # far above random rows
    kc, ks, sel, sc = _run(m, keys2, q, wt, 4000)
    np.testing.assert_array_equal(sel, top[:4000].astype(np.int32))
    np.testing.assert_array_equal(sel, oracle.index_topk(sc.astype(np.float64), 4000))


def test_index_duplicate_rows_straddle_the_boundary(m):
    # 40 copies of one key row: equal scores; k cuts through the copies, which
    # must then go to the smallest row indices
    say("index duplicates at the boundary")
    g = np.random.Generator(np.random.PCG64(32))
    keys = (g.standard_normal((2000, 128)) * 0.1).astype(np.float32)
    q = g.standard_normal((16, 128)).astype(np.float32)
    wt = np.abs(g.standard_normal(16)).astype(np.float32)
    dup = np.sort(g.choice(2000, 40, replace=False))
    keys[dup] = g.standard_normal(128).astype(np.float32) * 5.0  # far above the rest
    kc, ks, sel, sc = _run(m, keys, q, wt, 25)
    assert len(set(sc[dup].tolist())) == 1
    np.testing.assert_array_equal(sel, dup[:25].astype(np.int32))


def test_index_selection_feeds_the_gather_decode(m):
    # the indexer's rows drive mla8_decode_sel over a latent shadow
    say("index -> decode_sel")
    wl, wi = W.DSA, W.DSA_INDEX
    t = 8192
    g = np.random.Generator(np.random.PCG64(33))
    keys = g.standard_normal((t, 128)).astype(np.float32)
    q = g.standard_normal((64, 128)).astype(np.float32)
    wt = W.index_weights(wi)
    kc, ks, sel, sc = _run(m, keys, q, wt, 512)
    x = W.rows(wl, t)
    codes, scales = m.mla8_quantize_rows(dev(x), wl.lc, wl.rc)
    ql, qr = W.queries(wl)
    out, lse = m.mla8_decode_sel(codes, scales, t, wl.lc, wl.rc, dev(sel), dev(ql), dev(qr),
                                 wl.sm_scale)
    oc, os_ = oracle.quantize_rows(x)
    # 512 selected rows: the e4m3-lo score path, checked against its query reading
    qa, qb = oracle.query_lo8(ql, qr, wl.sm_scale)
    ro, rl = oracle.decode_sel(oc, os_, t, wl.lc, wl.rc, sel, qa, qb, wl.sm_scale)
    from tests.tolerance import check_attention
    check_attention(host(out), ro, host(lse), rl, "index -> decode_sel")


def test_index_threshold_many_bins_below_the_largest_key(m):
    # ten rows scaled by 1e30 put the largest keys ~790 first-digit bins above
    # the rest, so the candidate pass reads several 512-bin windows of the
    # histogram before it reaches the k-th key
    say("index: k-th key far below the largest")
    g = np.random.Generator(np.random.PCG64(35))
    keys = g.standard_normal((9000, 128)).astype(np.float32)
    big = np.sort(g.choice(9000, 10, replace=False))
    keys[big] *= np.float32(1e30)
    q = g.standard_normal((32, 128)).astype(np.float32)
    wt = np.abs(g.standard_normal(32)).astype(np.float32) / np.float32(8.0)
    kc, ks, sel, sc = _run(m, keys, q, wt, 300)
    ref = oracle.index_scores(kc, ks, q, wt)
    assert np.isfinite(ref).all() and ref.max() > 1e25
    _check(sel, sc, ref, _bound(kc, ks, q, wt), 300, "outlier rows")
    # the outlier rows with a positive score are all chosen
    assert set(big[sc[big] > 1e20].tolist()) <= set(sel.tolist())


def test_index_graph_replays_match_eager(m):
    # the bench replays captured indexer calls: every replay must reproduce the
    # eager selection and scores (the call clears its histogram and
    # largest-key words with a kernel of its own, so replays start clean)
    say("index under graph replay")
    g = np.random.Generator(np.random.PCG64(36))
    keys = g.standard_normal((30000, 128)).astype(np.float32)
    q = g.standard_normal((64, 128)).astype(np.float32)
    wt = (g.standard_normal(64) / 8).astype(np.float32)
    kc, ks = m.mla8_quantize_rows(dev(keys), 128, 0)
    qd, wd = dev(q), dev(wt)
    sel = torch.empty((2048,), dtype=torch.int32, device=DEV)
    sc = torch.empty((30000,), dtype=torch.float32, device=DEV)
    need = m.mla8_workspace_bytes(m.MLA8_OP_INDEX, 30000, 64, 1, 128)
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV)

    def call():
        m.mla8_index_topk(kc, ks, qd, wd, 2048, sel=sel, scores=sc, workspace=ws)

    call()
    ref_sel, ref_sc = host(sel).copy(), host(sc).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call()
    for r in range(4):
        sel.fill_(-1)
        sc.zero_()
        ws.fill_(0xAB)  # stale workspace contents must not matter
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(sel), ref_sel), r
        assert np.array_equal(host(sc).view(np.uint32), ref_sc.view(np.uint32)), r
        _ = (torch.ones(1000, device=DEV) * 2).sum().item()  # eager work between replays
    ref = oracle.index_scores(host(kc), host(ks), q, wt)
    _check(ref_sel, ref_sc, ref, _bound(host(kc), host(ks), q, wt), 2048, "graph replay")


def test_index_truncation_adversarial(m):
    """Every aligned group of 8 key/query positions holds one 448 x 448
    product and seven products of 4 to 7.6, below the group's truncation unit
    2^3, all positive: the fp8 MFMA drops the seven (about 2e-4 of A_t, ten
    times the typical bound); the scores stay within the contract bound and
    the selection within it of the fp64 one."""
    t, n_ih, k = 4096, 16, 256
    say(f"index truncation-adversarial t={t} n_ih={n_ih} k={k}")
    g = np.random.Generator(np.random.PCG64(77))
    small = np.array([2.0, 2.25, 2.5, 2.75], np.float32)
    keys = g.choice(small, (t, 128)).astype(np.float32)
    q = g.choice(small, (n_ih, 128)).astype(np.float32)
    big = 8 * np.arange(16) + g.integers(0, 8, 16)   # one position per group of 8
    keys[:, big] = 448.0
    q[:, big] = 448.0
    wt = (g.uniform(0.5, 1.5, n_ih) / n_ih).astype(np.float32)
    kc, ks, sel, sc = _run(m, keys, q, wt, k)
    assert np.all(ks == 1.0)   # amax 448: every code exact
    ref = oracle.index_scores(kc, ks, q, wt)
    a = _bound(kc, ks, q, wt, rel=1.0)
    rel_err = float((np.abs(sc.astype(np.float64) - ref) / a).max())
    say(f"  worst error {rel_err:.3g} of A_t (typical bound {REL:g}, contract {REL_CONTRACT:.3g})")
    _check(sel, sc, ref, _bound(kc, ks, q, wt, rel=REL_CONTRACT), k, "truncation-adversarial")
