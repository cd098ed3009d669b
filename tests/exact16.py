"""Exact references for the pins, built from definitions rather than from the
oracle: nearest-fp16 by search over the list of all fp16 values, integer
round-half-to-even of a rational, brute-force nearest code."""
import bisect
from fractions import Fraction

import numpy as np

_POS_BITS = np.arange(0, 0x7C00, dtype=np.uint16)               # +0 .. 65504
_POS_VALS = [Fraction(float(v)) for v in _POS_BITS.view(np.float16).astype(np.float64)]


def nearest_f16_bits(r):
    """fp16 bit pattern nearest to the rational r >= 0 (ties to the pattern
    with an even last bit; beyond the halfway point past 65504: +inf)."""
    r = Fraction(r)
    assert r >= 0
    top = _POS_VALS[-1]
    if r >= top + (Fraction(65536) - top) / 2:
        return 0x7C00
    i = bisect.bisect_left(_POS_VALS, r)
    if i < len(_POS_VALS) and _POS_VALS[i] == r:
        return int(_POS_BITS[i])
    lo, hi = i - 1, i
    if hi == len(_POS_VALS):                     # between 65504 and the halfway point
        return int(_POS_BITS[lo])
    dl, dh = r - _POS_VALS[lo], _POS_VALS[hi] - r
    if dl < dh:
        return int(_POS_BITS[lo])
    if dh < dl:
        return int(_POS_BITS[hi])
    return int(_POS_BITS[lo]) if _POS_BITS[lo] % 2 == 0 else int(_POS_BITS[hi])


def f16_units(bits):
    """fp16 values as exact integers in units of 2^-24 (int64), for finite inputs."""
    v = np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)
    return np.round(v * 2.0 ** 24).astype(np.int64)       # exact: v * 2^24 is an integer


def rne_div_clamp(X, S, Z):
    """round_half_even(X / S) clamped to [-Z, Z-1]; integer arithmetic (S > 0)."""
    X = np.asarray(X, np.int64)
    S = np.asarray(S, np.int64)
    q0 = np.floor_divide(X, S)
    rem = X - q0 * S                                      # 0 <= rem < S
    twice = 2 * rem
    up = (twice > S) | ((twice == S) & (q0 % 2 != 0))
    q = q0 + up.astype(np.int64)
    return np.clip(q, -Z, Z - 1)


def argmin_code(x, s, Z):
    """Brute force: the integer k in [-Z, Z-1] minimising |x - k*s| (exact in
    float64 for fp16 x, s and |k| <= 32), ties to the even k."""
    x = np.asarray(x, np.float64)[:, None]
    s = np.asarray(s, np.float64)[:, None] if np.ndim(s) else np.float64(s)
    ks = np.arange(-Z, Z, dtype=np.float64)[None, :]
    d = np.abs(x - ks * s)
    m = d.min(axis=1, keepdims=True)
    cand = d == m
    even = cand & (ks % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return (ks[0, pick]).astype(np.int64)
