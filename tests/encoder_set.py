"""The e4m3 encoder test set (tiny workload): 4096 f32 values.

Test input only.  The e4m3 magnitudes are generated from the bit layout named by
colibri PR #300's KV8-base commit (1 sign, 4 exponent bits with bias 7, 3
mantissa bits, finite range +/-448) so that this module depends on neither the
oracle nor the HIP library.
"""
from __future__ import annotations

import numpy as np

from fp8_mla_latent_amd.workloads import rng


def encoder_values(n: int = 4096, seed: int = 1) -> np.ndarray:
    """f32 test values for the e4m3 encoder: every e4m3 magnitude, every midpoint
    between neighbouring magnitudes and its f32 neighbours, the saturation edge,
    +/-0, f32 subnormals, +/-FLT_MIN, +/-inf, quiet and signalling NaNs of both
    signs, then seeded uniform values on [-600, 600] and log-uniform magnitudes.

    The e4m3 magnitudes are generated from the bit layout (1-4-3, bias 7) so that
    this module stays independent of both implementations."""
    mags = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            mags.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    mags = np.array(sorted(mags), np.float64)
    mids = (mags[:-1] + mags[1:]) / 2  # exact in f32: at most 5 significant bits
    vals = [mags, -mags, mids, -mids]
    m32 = mids.astype(np.float32)
    vals += [np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf))]
    edge = np.array([448, 448.00003, 463.99, 464, 464.00003, 465, 479, 480, 600, 1e30],
                    np.float32)
    vals += [edge, -edge]
    bits = np.array([0x00000000, 0x80000000,            # +0, -0
                     0x00000001, 0x007FFFFF, 0x00400000,  # f32 subnormals
                     0x80000001, 0x807FFFFF,
                     0x00800000, 0x80800000,              # +/-FLT_MIN
                     0x7F800000, 0xFF800000,              # +/-inf
                     0x7FC00000, 0xFFC00000,              # quiet NaNs
                     0x7F800001, 0xFFA00000],             # signalling NaNs
                    np.uint32)
    vals.append(bits.view(np.float32))
    base = np.concatenate([np.asarray(v, np.float32) for v in vals])
    g = rng(seed * 1000 + 900)
    rest = n - base.size
    half = rest // 2
    uni = g.uniform(-600.0, 600.0, size=half).astype(np.float32)
    logm = np.exp2(g.uniform(-12.0, 9.0, size=rest - half)) * g.choice([-1.0, 1.0], rest - half)
    out = np.concatenate([base, uni, logm.astype(np.float32)])
    assert out.size == n and out.dtype == np.float32
    return out
