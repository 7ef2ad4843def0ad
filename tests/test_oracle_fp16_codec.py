"""Pins of the oracle's fp16 conversions and INT2 codec.

The conversions are pinned to numpy's IEEE binary16 implementation (a library
routine); the codec is pinned to an exact-rational restatement of the rounding
rule (Python Fractions, round-half-even) on top of numpy's fp32 arithmetic, to
the closed-form special cases (constant group, exact arithmetic progression,
half-way ties) and to the worst-case error bound |x - x_hat| <= scale / 2.
"""
from fractions import Fraction

import numpy as np
import pytest


def test_h2d_all_patterns(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.h2d(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert np.signbit(oracle.h2d(0x8000)) and not np.signbit(oracle.h2d(0))


def _f2h_cases():
    r = np.random.default_rng(7)
    finite = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = finite[np.isfinite(finite)].astype(np.float32)
    pos = np.sort(finite[finite >= 0].astype(np.float64))
    pos = np.unique(pos)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)   # exact ties
    rand = (r.standard_normal(60000) *
            np.exp2(r.integers(-30, 18, 60000))).astype(np.float32)
    edge = np.array([65504, 65519.99, 65520, 65535, 1e9, 5.96e-8, 2.98e-8,
                     2.9802322e-08, 1e-9, 0.0, -0.0, 6.1035156e-05,
                     6.1035156e-05 * (1 - 2 ** -12)], np.float32)
    return np.concatenate([finite, mids, -mids, rand, edge])


def test_f2h_rne_matches_numpy(oracle):
    xs = _f2h_cases()
    ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f2h_rne(x) for x in xs], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (xs[bad[:5]], got[bad[:5]], ref[bad[:5]])


def _codec_ref(x16):
    """Restatement of the codec rule with exact rationals."""
    xf = x16.astype(np.float32)
    mn, mx = xf.min(), xf.max()
    s32 = np.float32(np.float32(mx - mn) / np.float32(3.0))
    sh = np.float16(s32)
    zh = np.float16(np.float32(mn) + np.float32(0.0))
    codes = []
    for xi in xf:
        if sh == 0:
            codes.append(0)
            continue
        d = np.float32(xi - np.float32(zh))
        q = Fraction(float(d)) / Fraction(float(sh))
        c = round(q)                      # Python rounds ties to even
        codes.append(int(min(max(c, 0), 3)))
    return (np.array(codes, np.uint8), int(np.array(sh).view(np.uint16)),
            int(np.array(zh).view(np.uint16)))


@pytest.mark.parametrize("G", [16, 32])
def test_codec_random_groups_vs_rational(oracle, G):
    r = np.random.default_rng(11)
    for trial in range(400):
        scale = np.exp2(r.integers(-12, 6))
        x = (r.standard_normal(G) * scale).astype(np.float16)
        if trial % 7 == 0:
            x[r.integers(0, G)] *= np.float16(10)       # outlier
        codes, s, z = oracle.quant_group(x)
        rc, rs, rz = _codec_ref(x)
        assert s == rs and z == rz
        assert np.array_equal(codes, rc), (x, codes, rc)


def test_codec_exhaustive_pairs_band(oracle):
    """Every (min, max) pair of fp16 values on a grid of the band [-4, 4],
    with the group's interior points at the quarter positions."""
    band = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    band = np.unique(band[np.isfinite(band) & (np.abs(band) <= 4)])
    sub = band[::97]
    checked = 0
    for i, a in enumerate(sub):
        for b in sub[i + 1::5]:
            t = np.linspace(float(a), float(b), 16)
            x = t.astype(np.float16)
            x[0], x[-1] = a, b
            codes, s, z = oracle.quant_group(x)
            rc, rs, rz = _codec_ref(x)
            assert (s, z) == (rs, rz) and np.array_equal(codes, rc)
            checked += 1
    assert checked > 5000


def test_codec_constant_group(oracle):
    x = np.full(16, 1.375, np.float16)
    codes, s, z = oracle.quant_group(x)
    assert s == 0 and np.all(codes == 0)
    assert oracle.dequant(0, s, z) == np.float32(1.375)


def test_codec_exact_progression(oracle):
    # z + c*s with exact fp16 s: codes 0..3 and exact reconstruction
    z, s = np.float16(-1.25), np.float16(0.375)
    vals = np.array([z + c * s for c in (0, 1, 2, 3)], np.float16)
    x = np.tile(vals, 4)
    codes, sb, zb = oracle.quant_group(x)
    assert np.array(s).view(np.uint16) == sb and np.array(z).view(np.uint16) == zb
    assert np.array_equal(codes, np.tile([0, 1, 2, 3], 4))
    for c, v in zip(codes, x):
        assert oracle.dequant(c, sb, zb) == np.float32(v)


def test_codec_half_way_ties_go_even(oracle):
    # min 0, max 3 -> scale exactly 1; 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    x = np.array([0, 3, 0.5, 1.5, 2.5, 1, 2, 0.25, 2.75] + [1] * 7,
                 np.float16)
    codes, s, z = oracle.quant_group(x)
    assert oracle.h2d(s) == 1.0 and oracle.h2d(z) == 0.0
    assert list(codes[:9]) == [0, 3, 0, 2, 2, 1, 2, 0, 3]


def test_codec_negative_zero_min_is_canonical(oracle):
    x = np.array([-0.0, 0.5, 1.0] + [0.25] * 13, np.float16)
    _, _, z = oracle.quant_group(x)
    assert z == 0x0000


def test_codec_error_bound(oracle):
    """|x - x_hat| <= s/2 (+ half an fp32 ulp of x_hat for the single rounding
    of the dequant add) wherever d = x - z is exact in fp32."""
    r = np.random.default_rng(3)
    for _ in range(300):
        x = (r.standard_normal(16) * np.exp2(r.integers(-6, 4))).astype(np.float16)
        codes, s, z = oracle.quant_group(x)
        sf, zf = oracle.h2d(s), oracle.h2d(z)
        for c, xi in zip(codes, x.astype(np.float64)):
            xh = float(oracle.dequant(c, s, z))
            if np.float32(xi) - np.float32(zf) != xi - zf:
                continue
            bound = sf / 2 + np.spacing(np.float32(abs(xh))) / 2
            assert abs(xi - xh) <= bound * (1 + 1e-12)


def test_dequant_single_rounding(oracle):
    r = np.random.default_rng(5)
    for _ in range(2000):
        s = np.float16(abs(r.standard_normal()) * 2.0 ** r.integers(-8, 4))
        z = np.float16(r.standard_normal() * 4)
        c = int(r.integers(0, 4))
        got = oracle.dequant(c, int(np.array(s).view(np.uint16)),
                             int(np.array(z).view(np.uint16)))
        ref = np.float32(Fraction(c) * Fraction(float(s)) + Fraction(float(z)))
        assert got == ref
