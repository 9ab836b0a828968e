"""GPU parity of the fused append + decode entry point (mla8_append_decode):
the same shadow bytes and the same attention as mla8_append followed by
mla8_decode, and the oracle's result, including fresh rows that straddle a row
chunk boundary and a full 64-row append that fills the shadow."""
from __future__ import annotations

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


def _run(m, w, t_total, n_new, cap=None, splits=0, seed=0):
    """Two shadows with the same t_total - n_new old rows: one takes
    append + decode, the other the fused call.  Returns both results and the
    oracle's."""
    cap = cap or t_total
    x = W.rows(w, t_total, seed_offset=seed)
    ql, qr = W.queries(w, seed_offset=seed)
    t_old = t_total - n_new
    shadows = []
    for _ in range(2):
        codes = torch.zeros((cap, w.d), dtype=torch.uint8, device=DEV)
        scales = torch.zeros((cap,), dtype=torch.float32, device=DEV)
        t = m.mla8_append(codes, scales, 0, dev(x[:t_old]), w.lc, w.rc)
        assert t == t_old
        shadows.append((codes, scales))
    (ca, sa), (cb, sb) = shadows
    t = m.mla8_append(ca, sa, t_old, dev(x[t_old:]), w.lc, w.rc)
    out_a, lse_a = m.mla8_decode(ca, sa, t, w.lc, w.rc, dev(ql), dev(qr), w.sm_scale,
                                 n_splits=splits)
    out_b, lse_b, tb = m.mla8_append_decode(cb, sb, t_old, dev(x[t_old:]), w.lc, w.rc,
                                            dev(ql), dev(qr), w.sm_scale, n_splits=splits)
    torch.cuda.synchronize()
    assert tb == t_total
    oc, os_ = oracle.quantize_rows(x)
    ro, rl = oracle.decode(oc, os_, t_total, w.lc, w.rc, ql, qr, w.sm_scale)
    return (ca, sa, out_a, lse_a), (cb, sb, out_b, lse_b), (oc, os_, ro, rl)


@pytest.mark.parametrize("n_new", [1, 3])
@pytest.mark.parametrize("w", [W.TINY, W.DSV3], ids=lambda w: w.name)
def test_append_decode_matches_append_then_decode(m, w, n_new):
    say(f"append_decode {w.name} n_new={n_new}")
    (ca, sa, oa, la), (cb, sb, ob, lb), (oc, os_, ro, rl) = _run(m, w, w.t_rows, n_new)
    t = w.t_rows
    assert np.array_equal(host(cb)[:t], oc), "fused append: codes differ from the oracle"
    assert np.array_equal(host(sb)[:t].view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(host(ca), host(cb)) and np.array_equal(host(sa), host(sb))
    # same kernels over the same bytes: identical results
    assert np.array_equal(host(oa), host(ob)) and np.array_equal(host(la), host(lb))
    check_attention(host(ob), ro, host(lb), rl, f"append_decode {w.name} n_new={n_new}",
                    outliers=w.outlier_frac > 0)


def test_append_decode_fresh_rows_in_an_early_tile(m):
    # one chunk of 128 rows: the fresh rows 97..99 lie in its second tile,
    # among the tiles whose loads go out before the streaming loop starts
    w = W.TINY
    say("append_decode fresh rows in tile 1")
    (ca, sa, oa, la), (cb, sb, ob, lb), (oc, os_, ro, rl) = _run(m, w, 100, 3)
    assert np.array_equal(host(cb)[:100], oc) and np.array_equal(host(sb)[:100], os_)
    assert np.array_equal(host(oa), host(ob)) and np.array_equal(host(la), host(lb))
    check_attention(host(ob), ro, host(lb), rl, "append_decode early tile")


def test_append_decode_rows_straddle_a_chunk_boundary(m):
    # 16 forced chunks of 256 rows over 3842 rows: fresh rows 3838..3841 fall
    # in chunks 14 (its fourth tile) and 15 (its first), each quantized by the
    # workgroups of its own chunk
    w = W.DSV3
    say("append_decode straddling chunk boundary")
    (ca, sa, oa, la), (cb, sb, ob, lb), (oc, os_, ro, rl) = _run(m, w, 3842, 4, splits=16)
    assert np.array_equal(host(cb), oc) and np.array_equal(host(sb), os_)
    assert np.array_equal(host(oa), host(ob)) and np.array_equal(host(la), host(lb))
    check_attention(host(ob), ro, host(lb), rl, "append_decode straddle", outliers=True)


def test_append_decode_full_64_rows_to_capacity(m):
    w = W.TINY
    say("append_decode 64 rows filling the shadow")
    (ca, sa, oa, la), (cb, sb, ob, lb), (oc, os_, ro, rl) = _run(m, w, 256, 64, cap=256)
    assert np.array_equal(host(cb), oc) and np.array_equal(host(sb), os_)
    check_attention(host(ob), ro, host(lb), rl, "append_decode 64 rows")
    # the shadow is full now: one more row is refused, nothing written
    x1 = W.rows(w, 1, seed_offset=9)
    ql, qr = W.queries(w)
    with pytest.raises(m.Mla8Error) as e:
        m.mla8_append_decode(cb, sb, 256, dev(x1), w.lc, w.rc, dev(ql), dev(qr), w.sm_scale)
    assert e.value.status == m.MLA8_E_CAPACITY


def test_append_decode_graph_replays_match_eager(m):
    # the bench replays a captured step; every replay must reproduce the eager
    # result (the fused append rewrites the same fresh row each time)
    w = W.DSV3
    say("append_decode under graph replay")
    t = 3000
    x = W.rows(w, t, seed_offset=4)
    ql, qr = W.queries(w, seed_offset=4)
    codes = torch.zeros((t, w.d), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((t,), dtype=torch.float32, device=DEV)
    assert m.mla8_append(codes, scales, 0, dev(x[:t - 1]), w.lc, w.rc) == t - 1
    fresh, qld, qrd = dev(x[t - 1:]), dev(ql), dev(qr)
    out = torch.empty((w.n_heads, w.lc), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.n_heads,), dtype=torch.float32, device=DEV)
    ws = torch.empty(m.mla8_workspace_bytes(m.MLA8_OP_DECODE, t, w.n_heads, 1, w.lc),
                     dtype=torch.uint8, device=DEV)

    def step():
        m.mla8_append_decode(codes, scales, t - 1, fresh, w.lc, w.rc, qld, qrd, w.sm_scale,
                             out=out, lse=lse, workspace=ws)

    step()
    ref_out, ref_lse = host(out).copy(), host(lse).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref_out), r
        assert np.array_equal(host(lse), ref_lse), r
        _ = (torch.ones(1000, device=DEV) * 2).sum().item()  # eager work between replays
    oc, os_ = oracle.quantize_rows(x)
    ro, rl = oracle.decode(oc, os_, t, w.lc, w.rc, ql, qr, w.sm_scale)
    check_attention(ref_out, ro, ref_lse, rl, "append_decode graph", outliers=True)
