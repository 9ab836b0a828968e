"""Pins for the oracle's indexer score and top-k (no GPU).

The page passage is the commit message of the B2 fp8 indexer score + top-k
kernel ("B1 Mixed FP8/BF16 FMHA first pass" site): the indexer query
quantized to fp8, the keys read as e4m3, dequantization by q_scale * k_scale,
ReLU, a weighted sum over the indexer heads, then top-k over the rows.  Each
test checks the oracle against something other than itself: a float64 numpy
computation on inputs the quantizer represents exactly, invariants of the
formula (scale homogeneity, linearity in the weights, the ReLU identities
relu(s) + relu(-s) = |s| and relu(s) - relu(-s) = s, row permutation), and a
pure-Python brute-force selection.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle

# e4m3-representable magnitudes well inside the normal range
_VALS = np.array([0.0, 0.5, 0.75, 1.0, 1.25, 1.5, 2.0, 3.0, 3.5, 5.0, 6.0, 7.0, 10.0, 12.0,
                  20.0, 28.0, 40.0, 64.0], np.float32)


def _exact_matrix(g, rows, cols):
    """Rows of e4m3-exact values, each with one entry of magnitude 448, so the
    row's scale is exactly 1 and its codes decode to the values themselves."""
    x = g.choice(_VALS, size=(rows, cols)) * g.choice([-1.0, 1.0], size=(rows, cols))
    x = x.astype(np.float32)
    for r in range(rows):
        x[r, g.integers(cols)] = np.float32(448.0) * g.choice([-1.0, 1.0])
    return x


def _closed_form(q, k, w, qscale=None, kscale=None):
    s = k.astype(np.float64) @ q.astype(np.float64).T  # [T, n_ih]
    if qscale is not None:
        s = s * qscale[None, :]
    if kscale is not None:
        s = s * kscale[:, None]
    return np.maximum(s, 0.0) @ w.astype(np.float64)


def test_index_scores_exact_inputs_closed_form():
    g = np.random.Generator(np.random.PCG64(71))
    n_ih, ihd, t = 3, 16, 9
    q = _exact_matrix(g, n_ih, ihd)
    k = _exact_matrix(g, t, ihd)
    kc, ks = oracle.quantize_rows(k)
    assert np.all(ks == 1.0) and np.array_equal(oracle.dec(kc), k.astype(np.float64))
    w = g.standard_normal(n_ih).astype(np.float32)
    got = oracle.index_scores(kc, ks, q, w)
    want = _closed_form(q, k, w)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-9)
    # every head contributes on some row, and ReLU drops some (head, row) pairs
    s = k.astype(np.float64) @ q.astype(np.float64).T
    assert (s > 0).any() and (s < 0).any()


def test_index_scores_both_scales_multiply():
    g = np.random.Generator(np.random.PCG64(72))
    n_ih, ihd, t = 4, 32, 12
    q = _exact_matrix(g, n_ih, ihd)
    k = _exact_matrix(g, t, ihd)
    a = g.integers(-6, 4, size=t)      # key row t scaled by 2^a_t
    b = g.integers(-5, 3, size=n_ih)   # query head j scaled by 2^b_j
    k2 = (k * np.exp2(a)[:, None]).astype(np.float32)
    q2 = (q * np.exp2(b)[:, None]).astype(np.float32)
    kc, ks = oracle.quantize_rows(k2)
    np.testing.assert_array_equal(ks, np.exp2(a).astype(np.float32))
    w = g.uniform(0.1, 1.0, n_ih).astype(np.float32)
    got = oracle.index_scores(kc, ks, q2, w)
    want = _closed_form(q, k, w, qscale=np.exp2(b), kscale=np.exp2(a))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-9)


def _random_case(seed, n_ih=8, ihd=64, t=40):
    g = np.random.Generator(np.random.PCG64(seed))
    kc, ks = oracle.quantize_rows(g.standard_normal((t, ihd)).astype(np.float32))
    q = g.standard_normal((n_ih, ihd)).astype(np.float32)
    return g, kc, ks, q


def test_index_scores_linear_in_weights_and_nonnegative_per_head():
    g, kc, ks, q = _random_case(73)
    # multiples of 1/8: w1 + w2 is exact in f32
    w1 = (g.integers(-16, 17, q.shape[0]) / 8.0).astype(np.float32)
    w2 = (g.integers(-16, 17, q.shape[0]) / 8.0).astype(np.float32)
    i1 = oracle.index_scores(kc, ks, q, w1)
    i2 = oracle.index_scores(kc, ks, q, w2)
    i12 = oracle.index_scores(kc, ks, q, (w1 + w2).astype(np.float32))
    np.testing.assert_allclose(i12, i1 + i2, rtol=1e-12, atol=1e-12 * np.abs(i1).max())
    np.testing.assert_array_equal(oracle.index_scores(kc, ks, q, -w1), -i1)
    for j in range(q.shape[0]):
        e = np.zeros(q.shape[0], np.float32)
        e[j] = 1.0
        assert (oracle.index_scores(kc, ks, q, e) >= 0).all()


def test_index_scores_relu_identities():
    # head 1 is head 0 negated: the quantizer is sign-symmetric, so the two
    # heads' dequantized dot products are s and -s exactly
    g, kc, ks, q1 = _random_case(74, n_ih=1)
    q = np.concatenate([q1, -q1]).astype(np.float32)
    s_abs = oracle.index_scores(kc, ks, q, np.array([1.0, 1.0], np.float32))
    s_sgn = oracle.index_scores(kc, ks, q, np.array([1.0, -1.0], np.float32))
    np.testing.assert_array_equal(s_abs, np.abs(s_sgn))
    assert (s_sgn > 0).any() and (s_sgn < 0).any()
    # and s itself is the dequantized dot product
    deq_k = oracle.dequant(kc, ks)
    qc, qs = oracle.quantize_rows(q1)
    deq_q = oracle.dequant(qc, qs)[0]
    np.testing.assert_allclose(s_sgn, deq_k @ deq_q, rtol=1e-12, atol=1e-12)


def test_index_scores_row_permutation():
    g, kc, ks, q = _random_case(75)
    w = g.standard_normal(q.shape[0]).astype(np.float32)
    perm = g.permutation(kc.shape[0])
    np.testing.assert_array_equal(oracle.index_scores(kc[perm], ks[perm], q, w),
                                  oracle.index_scores(kc, ks, q, w)[perm])


def _brute_topk(scores, k):
    """Pick the best remaining row k times: non-NaN first, larger score, then
    the smaller index."""
    left = list(range(len(scores)))
    out = []
    for _ in range(min(k, len(scores))):
        best = None
        for t in left:
            s = scores[t]
            key = (0 if math.isnan(s) else 1, -math.inf if math.isnan(s) else s, -t)
            if best is None or key > best[0]:
                best = (key, t)
        out.append(best[1])
        left.remove(best[1])
    return sorted(out)


@pytest.mark.parametrize("case", [
    ([1.0, 3.0, 3.0, 3.0, 2.0], 2),                 # ties go to the smaller index
    ([math.nan, 1.0, math.nan, 0.0], 3),            # NaN below every other score
    ([math.nan, 1.0, math.nan, 0.0], 2),
    ([-0.0, 0.0, -0.0], 1),                         # signed zeros are equal
    ([5.0, -math.inf, math.inf, math.nan, 2.0], 4),
    ([0.5, 0.25], 7),                               # T <= k: every row
])
def test_topk_small_cases(case):
    s, k = case
    got = oracle.index_topk(np.array(s), k)
    assert got.tolist() == _brute_topk(s, k)


def test_topk_random_against_brute_force():
    g = np.random.Generator(np.random.PCG64(76))
    for trial in range(20):
        t = int(g.integers(1, 60))
        s = np.round(g.standard_normal(t), 1)  # rounding makes ties common
        s[g.random(t) < 0.1] = np.nan
        k = int(g.integers(1, 70))
        assert oracle.index_topk(s, k).tolist() == _brute_topk(s.tolist(), k), trial


def test_topk_zero_weights_select_the_first_rows():
    g, kc, ks, q = _random_case(77)
    s = oracle.index_scores(kc, ks, q, np.zeros(q.shape[0], np.float32))
    assert (s == 0).all()
    assert oracle.index_topk(s, 5).tolist() == [0, 1, 2, 3, 4]
