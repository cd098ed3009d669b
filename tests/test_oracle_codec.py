"""Pins of the oracle's fp16 codec and 8-bit format against references that do
not come from the oracle: numpy's IEEE binary16 conversion (a library
routine), exact rational arithmetic, and the e5m2 format definition.

The 8-bit format is the high byte of the fp16 pattern (the page's FP8, stored unsigned)
on the ExLlamaV2 cache page (Description of fp16_to_fp8 / fp8_to_fp16).

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

ALL16 = np.arange(65536, dtype=np.uint16)


def test_decode_exhaustive_vs_numpy():
    got = oracle.f16_decode(ALL16)
    ref = ALL16.view(np.float16).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # signed zero is kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0x0000])


def test_encode_roundtrip_exhaustive():
    vals = ALL16.view(np.float16).astype(np.float64)
    fin = ~np.isnan(vals)
    assert (oracle.f16_encode_rne(vals[fin]) == ALL16[fin]).all()
    assert (oracle.f16_encode_rne(np.array([np.nan])) & 0x7C00) == 0x7C00


def _midpoints():
    """Exact midpoints between consecutive non-negative fp16 values, and their
    immediate float64 neighbours: the inputs where rounding decides."""
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = np.arange(1, 0x7C01, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt[-1] = 65536.0                            # the next binade's first value
    mid = (pos + nxt) / 2                        # exact in float64
    v = np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])
    return np.concatenate([v, -v])


def test_encode_vs_numpy_at_rounding_boundaries():
    v = _midpoints()
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert (oracle.f16_encode_rne(v) == ref).all()


def test_encode_vs_numpy_random():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-30, 17, size=400_000))
    v = mag * rng.choice([-1.0, 1.0], size=mag.size)
    v32 = rng.standard_normal(200_000).astype(np.float32).astype(np.float64) * 1e3
    for arr in (v, v32):
        with np.errstate(over="ignore"):
            ref = arr.astype(np.float16).view(np.uint16)
        assert (oracle.f16_encode_rne(arr) == ref).all()


def test_encode_overflow_threshold():
    # 65504 is the largest finite value; the halfway point to 65536 is 65520.
    assert oracle.f16_encode_rne(np.array([65504.0, 65519.999, 65520.0, -65520.0])).tolist() == \
        [0x7BFF, 0x7BFF, 0x7C00, 0xFC00]


# ---------------------------------------------------------------- 8-bit (e5m2 truncation)
def _e5m2_value(byte):
    """Value of an e5m2 byte from the format definition: 1 sign bit, 5
    exponent bits with bias 15, 2 mantissa bits, subnormals at exponent 0."""
    s = -1 if byte & 0x80 else 1
    e = (byte >> 2) & 0x1F
    m = byte & 3
    if e == 0x1F:
        return s * float("inf") if m == 0 else float("nan")
    if e == 0:
        return s * Fraction(m, 4) * Fraction(1, 2 ** 14)
    return s * (1 + Fraction(m, 4)) * Fraction(2) ** (e - 15)


def test_fp8_is_high_byte_of_memory_image():
    # little-endian fp16: the high byte is the second byte in memory
    got = oracle.fp8_from_f16(ALL16)
    assert (got == ALL16.view(np.uint8)[1::2]).all()


def test_fp8_truncates_toward_zero():
    """Every finite fp16 maps to the e5m2 value of largest magnitude not
    exceeding it (same sign), i.e. truncation toward zero."""
    e5 = {b: _e5m2_value(b) for b in range(256)}
    pos_bytes = sorted((b for b in range(0x7C)), key=lambda b: e5[b])
    pos_vals = [e5[b] for b in pos_bytes]
    got = oracle.fp8_from_f16(ALL16)
    vals = ALL16.view(np.float16).astype(np.float64)
    for h in range(65536):
        x = vals[h]
        if not np.isfinite(x):
            continue
        ax = Fraction(abs(x))
        # largest e5m2 magnitude <= |x|
        best = max(i for i, pv in enumerate(pos_vals) if pv <= ax) if ax > 0 else 0
        want = pos_bytes[best] | (0x80 if (h & 0x8000) else 0)
        if ax == 0:
            want = 0x80 if (h & 0x8000) else 0x00
        assert got[h] == want, hex(h)


def test_fp8_back_and_roundtrip():
    b = np.arange(256, dtype=np.uint8)
    back = oracle.f16_from_fp8(b)
    # widening is exact: the fp16 value equals the e5m2 value of the byte
    for i in range(256):
        v = back.view(np.float16)[i].astype(np.float64)
        ref = _e5m2_value(i)
        if isinstance(ref, float) and np.isnan(ref):
            assert np.isnan(v)
        else:
            assert v == float(ref)
    rt = oracle.f16_from_fp8(oracle.fp8_from_f16(ALL16))
    assert (rt == (ALL16 & 0xFF00)).all()


@pytest.mark.parametrize("h,want", [(0x7C01, 0x7C), (0x3C00, 0x3C), (0x8001, 0x80), (0x3BFF, 0x3B)])
def test_fp8_edge_patterns(h, want):
    # 0x7C01 (a NaN with payload only in the low byte) becomes +Inf's byte;
    # 1.0 keeps its byte; the smallest negative subnormal truncates to -0.
    assert int(oracle.fp8_from_f16(np.array([h], np.uint16))[0]) == want
