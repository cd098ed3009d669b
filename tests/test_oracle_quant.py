"""Pins of the oracle's block quantization, dequantization and bit packing.

The ExLlamaV2 cache page (Description of fp16_to_q_kv / q_to_fp16_kv; I/O
Contract: k_scales / v_scales hold one scale factor per quantization block,
wbits is 4 or 6) fixes the operation but not the numerics; the readings used
(32-element blocks along head_dim, absmax / (2^(b-1)-1) in fp32 stored as fp16,
round-half-to-even codes against the stored scale clamped to
[-2^(b-1), 2^(b-1)-1], offset-binary storage, little-endian bit stream
packing) are checked here against exact arithmetic and brute force.

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact16 import argmin_code, f16_units, nearest_f16_bits, rne_div_clamp

POS_FINITE = np.arange(0, 0x7C00, dtype=np.uint16)
ALL_FINITE = np.concatenate([POS_FINITE, POS_FINITE | 0x8000])


def QZ(wbits):
    return (1 << (wbits - 1)) - 1, 1 << (wbits - 1)


# ---------------------------------------------------------------- scale
@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_scale_equals_exact_rational_rounding(wbits):
    """fp32 divide then fp16 rounding == single correct rounding of the exact
    rational a/Q, for every finite fp16 absmax."""
    Q, _ = QZ(wbits)
    got = oracle.scale_from_absmax(POS_FINITE, wbits)
    vals = POS_FINITE.view(np.float16).astype(np.float64)
    want = np.array([nearest_f16_bits(Fraction(float(a)) / Q) for a in vals], np.uint16)
    assert (got == want).all()


@pytest.mark.parametrize("wbits,n_zero,n_sub", [(4, 3, 3836), (6, 15, 6064), (8, 63, 8112)])
def test_scale_underflow_counts(wbits, n_zero, n_sub):
    s = oracle.scale_from_absmax(POS_FINITE, wbits)
    assert int(((s == 0) & (POS_FINITE != 0)).sum()) == n_zero
    assert int(((s > 0) & (s < 0x0400)).sum()) == n_sub


# ---------------------------------------------------------------- codes
@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_normal_scale_never_needs_the_clamp(wbits):
    """For every finite absmax a whose stored scale s16 is a normal fp16,
    a / s16 < Q + 1/2 exactly: every element of such a block rounds into
    [-Q, Q] without clamping (the clamp only acts under subnormal scales)."""
    Q, _ = QZ(wbits)
    s = oracle.scale_from_absmax(POS_FINITE, wbits)
    normal = s >= 0x0400
    A = f16_units(POS_FINITE[normal])
    S = f16_units(s[normal])
    assert (2 * A < (2 * Q + 1) * S).all()
    assert normal.sum() > 20000


def _scale_sample():
    """Every subnormal scale, every 16th normal scale, and all scales with an
    all-ones or all-zeros mantissa (binade edges)."""
    s = np.arange(1, 0x7C00, dtype=np.uint16)
    pick = (s < 0x0400) | (s % 16 == 0) | ((s & 0x3FF) == 0x3FF) | ((s & 0x3FF) == 0)
    return s[pick]


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_codes_exact_integer_rounding(wbits):
    """For all finite fp16 x and a wide sample of positive fp16 scales, the
    oracle's fp32 path equals integer round-half-even of X/S, clamped."""
    _, Z = QZ(wbits)
    X = f16_units(ALL_FINITE)
    for s in _scale_sample():
        u = oracle.quant_elems(ALL_FINITE, int(s), wbits).astype(np.int64)
        S = int(f16_units(np.array([s], np.uint16))[0])
        want = rne_div_clamp(X, S, Z) + Z
        assert (u == want).all(), hex(int(s))


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_codes_bruteforce_argmin(wbits):
    """Nearest representable multiple k*s, k in [-Z, Z-1], ties to even k, on
    every finite x for a handful of scales, including ones with exact ties."""
    _, Z = QZ(wbits)
    xv = ALL_FINITE.view(np.float16).astype(np.float64)
    for s in [0x0001, 0x0003, 0x00FF, 0x0400, 0x2E66, 0x3C00, 0x3555, 0x4248, 0x7092, 0x7BFF]:
        sv = float(np.uint16(s).view(np.float16))
        u = oracle.quant_elems(ALL_FINITE, s, wbits).astype(np.int64)
        want = argmin_code(xv, sv, Z) + Z
        assert (u == want).all(), hex(s)


def test_zero_scale_gives_zero_code():
    for wbits in (4, 6, 8):
        _, Z = QZ(wbits)
        u = oracle.quant_elems(ALL_FINITE, 0, wbits)
        assert (u == Z).all()


# ---------------------------------------------------------------- dequant
@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_dequant_exhaustive_vs_numpy(wbits):
    _, Z = QZ(wbits)
    u = np.arange(1 << wbits, dtype=np.uint8)
    for s in ALL_FINITE[::1]:
        got = oracle.dequant_elems(u, int(s), wbits)
        prod = (u.astype(np.float64) - Z) * float(np.uint16(s).view(np.float16))   # exact
        with np.errstate(over="ignore"):
            want = prod.astype(np.float16).view(np.uint16)
        assert (got == want).all(), hex(int(s))


def test_dequant_overflow_at_top_of_range():
    # absmax 65504: Q4 scale 9360 and 7*9360 = 65520 rounds to +inf; Q6 2114*31 = 65534 -> +inf
    for wbits, s_bits in [(4, 0x7092), (6, 0x6821)]:
        Q, Z = QZ(wbits)
        assert oracle.scale_from_absmax(np.array([0x7BFF], np.uint16), wbits)[0] == s_bits
        out = oracle.dequant_elems(np.array([Z + Q], np.uint8), s_bits, wbits)
        assert out[0] == 0x7C00


# ---------------------------------------------------------------- packing
def _read_golden_pack():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "pack_vectors.txt")
    cases = []
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            wb, codes, hexbytes = line.split("|")
            cases.append((int(wb), [int(c) for c in codes.split()], bytes.fromhex(hexbytes.strip())))
    return cases


def test_pack_golden_vectors():
    cases = _read_golden_pack()
    assert len(cases) >= 8
    for wbits, codes, want in cases:
        got = oracle.pack_bits(np.array(codes, np.uint8), wbits).tobytes()
        assert got == want, (wbits, codes)
        assert oracle.unpack_bits(np.frombuffer(want, np.uint8), len(codes), wbits).tolist() == codes


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_pack_equals_big_integer(wbits):
    """The stream equals the little-endian bytes of sum_j u_j * 2^(b*j)."""
    rng = np.random.default_rng(11)
    for n in (8, 16, 32, 48, 1024):
        if (n * wbits) % 8:
            continue
        u = rng.integers(0, 1 << wbits, size=n).astype(np.uint8)
        big = 0
        for j, c in enumerate(u.tolist()):
            big += c << (wbits * j)
        want = big.to_bytes(n * wbits // 8, "little")
        assert oracle.pack_bits(u, wbits).tobytes() == want
        assert (oracle.unpack_bits(oracle.pack_bits(u, wbits), n, wbits) == u).all()


def test_walking_bit_q6():
    for j in range(16):
        for k in range(6):
            u = np.zeros(16, np.uint8)
            u[j] = 1 << k
            p = oracle.pack_bits(u, 6)
            bit = 6 * j + k
            want = np.zeros(12, np.uint8)
            want[bit // 8] = 1 << (bit % 8)
            assert (p == want).all()


# ---------------------------------------------------------------- block invariants
def _round_trip_ok(x_bits, s16, u, xq_bits, wbits):
    """|x - x'| <= s/2 + ulp16(x')/2 unless the code was clamped or x' is inf.
    A scale that underflowed to 0 (absmax/Q below half the smallest subnormal)
    gives x' = 0 with |x| <= Q * 2^-25."""
    Q, Z = QZ(wbits)
    x = x_bits.view(np.float16).astype(np.float64)
    xq = xq_bits.view(np.float16).astype(np.float64)
    s = float(np.uint16(s16).view(np.float16))
    if s == 0:
        return bool((xq == 0).all() and (np.abs(x) <= Q * 2.0 ** -25).all())
    q = u.astype(np.int64) - Z
    clamped = ((q == -Z) | (q == Z - 1)) & (np.abs(x) > (Z - 0.5) * s)
    ok = np.isinf(xq) | clamped
    ulp = np.zeros_like(xq)
    fin = np.isfinite(xq)                   # infinite x' is accepted above
    ulp[fin] = np.spacing(np.abs(xq[fin]).astype(np.float16)).astype(np.float64)
    ok |= np.abs(x - xq) <= s / 2 + ulp / 2
    return ok.all()


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_block_invariants_random(wbits):
    Q, Z = QZ(wbits)
    rng = np.random.default_rng(5 + wbits)
    for trial in range(3000):
        scale = 2.0 ** rng.uniform(-20, 15)
        # finite inputs only (non-finite values are outside the contract)
        x = np.clip(rng.standard_normal(32) * scale, -65504, 65504).astype(np.float16)
        if trial % 50 == 0:
            x[:] = 0
        xb = x.view(np.uint16)
        s16, u = oracle.quant_block(xb, wbits)
        q = u.astype(np.int64) - Z
        assert ((q >= -Z) & (q <= Z - 1)).all()
        a = np.abs(x.astype(np.float64)).max()
        if a == 0:
            assert s16 == 0 and (u == Z).all()
            assert (oracle.dequant_elems(u, s16, wbits) == 0).all()    # +0
            continue
        if s16 >= 0x0400:                                  # normal scale: no clamping
            assert np.abs(q).max() == Q
            assert (np.abs(q) <= Q).all()
        xq = oracle.dequant_elems(u, s16, wbits)
        assert _round_trip_ok(xb, s16, u, xq, wbits)


ALPHABET = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0003, 0x000A, 0x03FF, 0x0400,
                     0x3800, 0xB800, 0x3C00, 0xBC00, 0x3E00, 0x4200, 0x4700, 0xC700,
                     0x4900, 0x5640, 0x3555, 0x7BFF, 0xFBFF, 0x1234, 0x2E66, 0x4B80],
                    np.uint16)


@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_tiny_blocks_bruteforce(wbits):
    """Every block of length 1..3 over a 24-value alphabet (zeros of both signs,
    subnormals, values that make exact ties, +-65504): scale = correctly rounded
    absmax/Q, codes = brute-force nearest multiple, invariants hold."""
    Q, Z = QZ(wbits)
    av = ALPHABET.view(np.float16).astype(np.float64)
    for L in (1, 2, 3):
        for idx in itertools.product(range(len(ALPHABET)), repeat=L):
            xb = ALPHABET[list(idx)]
            s16, u = oracle.quant_block(xb, wbits)
            a = max(abs(av[i]) for i in idx)
            assert s16 == nearest_f16_bits(Fraction(a) / Q)
            sv = float(np.uint16(s16).view(np.float16))
            if sv == 0:
                assert (u == Z).all()
            else:
                assert (u.astype(np.int64) == argmin_code(av[list(idx)], sv, Z) + Z).all()
            xq = oracle.dequant_elems(u, s16, wbits)
            assert _round_trip_ok(xb, s16, u, xq, wbits)


def test_clamp_example_subnormal_scale():
    # absmax 10 * 2^-24 at 4 bits: scale rounds to 2^-24, 10 clamps to 7 (u = 15)
    s16, u = oracle.quant_block(np.array([0x000A, 0x0000], np.uint16), 4)
    assert s16 == 0x0001 and u.tolist() == [15, 8]


# ---------------------------------------------------------------- rows
@pytest.mark.parametrize("wbits", [4, 6, 8])
def test_rows_compose_blocks_and_stream(wbits):
    """A token row is its 32-element blocks quantized independently, scales in
    block order, and all codes of the row in one bit stream."""
    rng = np.random.default_rng(3)
    for R in (32, 96, 160, 1024, 4128):
        x = (rng.standard_normal((2, R)) * 3).astype(np.float16)
        codes, scales = oracle.quant_rows(x, wbits)
        assert codes.shape == (2, R * wbits // 8) and scales.shape == (2, R // 32)
        for r in range(2):
            us = []
            for b in range(R // 32):
                s16, u = oracle.quant_block(x[r, 32 * b:32 * b + 32].view(np.uint16), wbits)
                assert scales[r, b] == s16
                us.append(u)
            assert (codes[r] == oracle.pack_bits(np.concatenate(us), wbits)).all()
        back = oracle.dequant_rows(codes, scales, wbits)
        for r in range(2):
            for b in range(R // 32):
                want = oracle.dequant_elems(
                    oracle.unpack_bits(codes[r], R, wbits)[32 * b:32 * b + 32], scales[r, b], wbits)
                assert (back[r, 32 * b:32 * b + 32] == want).all()
