"""Comparison helpers shared by the GPU parity tests.

Attention tolerance (stated for the absorbed fp8 decode path): per (query, head)
output vector, max_k |gpu - ref| <= 1e-4 + 2e-3 * max_k |ref|, where ref is the
fp64 oracle run on the same e4m3 bytes and scales.  The per-vector (normwise)
form is used because near-tied, near one-hot heads (rows with outlier amax)
make single small elements ill-conditioned even for exact f32 arithmetic.
lse is checked to |gpu - ref| <= 1e-4 + 2e-3 * |ref|.
"""
from __future__ import annotations

import numpy as np

ABS = 1e-4
REL = 2e-3


def check_attention(out_gpu, out_ref, lse_gpu=None, lse_ref=None, what=""):
    g = np.asarray(out_gpu, np.float64).reshape(-1, out_ref.shape[-1])
    r = np.asarray(out_ref, np.float64).reshape(-1, out_ref.shape[-1])
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r).max(1)
    bar = ABS + REL * np.abs(r).max(1)
    worst = float((err / bar).max()) if err.size else 0.0
    bad = np.flatnonzero(err > bar)
    assert bad.size == 0, (f"{what}: {bad.size} of {err.size} vectors out of tolerance; "
                           f"worst err/bar {worst:.3f} at vector {int(np.argmax(err / bar))}")
    if lse_ref is not None:
        lg = np.asarray(lse_gpu, np.float64).reshape(-1)
        lr = np.asarray(lse_ref, np.float64).reshape(-1)
        inf = np.isneginf(lr)
        assert np.array_equal(np.isneginf(lg), inf), f"{what}: lse -inf mismatch"
        d = np.abs(lg[~inf] - lr[~inf])
        assert np.all(d <= ABS + REL * np.abs(lr[~inf])), f"{what}: lse max err {d.max()}"
    return worst
