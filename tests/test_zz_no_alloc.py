"""GPU check of mla8_append_decode_noalloc (the entry point that allocates
nothing: its split-T partials live in the library's static device scratch)
against mla8_append_decode with a caller workspace, through the C ABI: two
calls in a row on the same GPU, the second with a smaller input, each with
identical shadow bytes and bit-identical attention output, and both within
the oracle's tolerance.  The second call also shows that what the first left
in the shared scratch does not leak into it."""
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


def _step_both(m, t_old, n_new, h, seed):
    """The DeepSeek-V3 row shape (lc 512, rc 64, 1 % of rows x50): two shadows
    of t_old rows; one takes the fresh rows through mla8_append_decode with a
    workspace, the other through mla8_append_decode_noalloc."""
    w = W.DSV3
    x = W.rows(w, t_old + n_new, seed_offset=seed)
    ql, qr = W.queries(w, seed_offset=seed)
    ql, qr = ql[:h], qr[:h]
    shadows = []
    for _ in range(2):
        codes = torch.zeros((t_old + n_new + 3, w.d), dtype=torch.uint8, device=DEV)
        scales = torch.zeros((t_old + n_new + 3,), dtype=torch.float32, device=DEV)
        assert m.mla8_append(codes, scales, 0, dev(x[:t_old]), w.lc, w.rc) == t_old
        shadows.append((codes, scales))
    (ca, sa), (cb, sb) = shadows
    fresh, qld, qrd = dev(x[t_old:]), dev(ql), dev(qr)
    out_a, lse_a, ta = m.mla8_append_decode(ca, sa, t_old, fresh, w.lc, w.rc, qld, qrd,
                                            w.sm_scale)
    out_b = torch.empty((h, w.lc), dtype=torch.float32, device=DEV)
    lse_b = torch.empty((h,), dtype=torch.float32, device=DEV)
    tb = m.mla8_append_decode_noalloc(cb, sb, t_old, fresh, w.lc, w.rc, qld, qrd, w.sm_scale,
                                      out_b, lse_b)
    assert ta == tb == t_old + n_new
    assert np.array_equal(host(ca), host(cb)) and np.array_equal(host(sa), host(sb))
    assert np.array_equal(host(out_a), host(out_b)), "noalloc output differs"
    assert np.array_equal(host(lse_a), host(lse_b)), "noalloc lse differs"
    t = t_old + n_new
    oc, os_ = oracle.quantize_rows(x)
    assert np.array_equal(host(cb)[:t], oc)
    ro, rl = oracle.decode(oc, os_, t, w.lc, w.rc, ql, qr, w.sm_scale)
    return check_attention(host(out_b), ro, host(lse_b), rl, f"noalloc t={t} h={h}",
                           outliers=True)


def test_noalloc_two_calls_second_smaller(m):
    say("noalloc: call 1, T=6000 (5997 + 3 fresh rows), 128 heads")
    w1 = _step_both(m, 5997, 3, 128, seed=21)
    say(f"  worst err/bar {w1:.4f}")
    say("noalloc: call 2, T=700 (699 + 1 fresh row), 16 heads")
    w2 = _step_both(m, 699, 1, 16, seed=22)
    say(f"  worst err/bar {w2:.4f}")


def test_noalloc_refuses_beyond_scratch(m):
    w = W.DSV3
    t = 262144
    codes = torch.zeros((t, w.d), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((t,), dtype=torch.float32, device=DEV)
    x = torch.zeros((1, w.d), dtype=torch.float32, device=DEV)
    q = torch.zeros((64, w.lc), dtype=torch.float32, device=DEV)
    qr = torch.zeros((64, w.rc), dtype=torch.float32, device=DEV)
    out = torch.empty((64, w.lc), dtype=torch.float32, device=DEV)
    with pytest.raises(m.Mla8Error) as e:
        m.mla8_append_decode_noalloc(codes, scales, t - 1, x, w.lc, w.rc, q, qr, 0.1, out,
                                     n_splits=1000)
    assert e.value.status == m.MLA8_E_SCRATCH
    assert not host(codes)[t - 1].any()  # nothing written
