"""Independent brute-force e4m3 helpers used to pin the oracle (test-only).

The table of e4m3 values comes from torch's float8_e4m3fn decoding of the 256
bytes, a library routine that shares nothing with the oracle.  Encoding is the
definition itself: the nearest finite e4m3 magnitude, ties to the even code,
anything at or above 448 saturates, NaN -> 0x00, the sign bit is copied.
"""
from __future__ import annotations

import numpy as np
import torch


def torch_decode_table() -> np.ndarray:
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


_TAB = torch_decode_table()
MAGS = _TAB[:0x7F].copy()          # codes 0x00..0x7E, increasing magnitudes
assert np.all(np.diff(MAGS) > 0)


def encode_bruteforce(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float32)
    a = np.abs(x.astype(np.float64))
    nan = np.isnan(x)
    a_safe = np.where(nan, 0.0, a)
    hi = np.searchsorted(MAGS, a_safe, side="left")      # first magnitude >= a
    hi = np.clip(hi, 0, MAGS.size - 1)
    lo = np.clip(hi - 1, 0, MAGS.size - 1)
    d_lo = a_safe - MAGS[lo]
    d_hi = MAGS[hi] - a_safe
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a_safe >= MAGS[-1], 0x7E, code)       # saturation at 448
    code = np.where(a_safe <= MAGS[0], 0, code)
    sign = np.signbit(x)
    code = np.where(sign, code | 0x80, code)
    code = np.where(nan, 0, code)
    return code.astype(np.uint8)


def half_gap(code: np.ndarray) -> np.ndarray:
    """Half the distance from |dec(code)| to its nearer neighbour on either side."""
    c = np.asarray(code, np.int64) & 0x7F
    up = MAGS[np.minimum(c + 1, 0x7E)] - MAGS[c]
    dn = MAGS[c] - MAGS[np.maximum(c - 1, 0)]
    up = np.where(c == 0x7E, dn, up)
    dn = np.where(c == 0, up, dn)
    return np.maximum(up, dn) / 2
