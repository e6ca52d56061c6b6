"""Pins of the oracle's OCP E4M3FN codec against values that do not come from the oracle:
the hand-written spot table (tests/golden/e4m3_spot.txt), exact rationals, exhaustive search
over the code table, and torch's float8_e4m3fn conversion (a library routine)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spot.txt")


def _spot_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        rows.append((float(parts[0]), int(parts[1], 16)))
    return rows


def test_decode_closed_forms():
    # values written from the format definition, not from the table builder
    assert e4m3.DECODE[0x7E] == 448.0
    assert e4m3.DECODE[0x08] == 2.0 ** -6
    assert e4m3.DECODE[0x01] == 2.0 ** -9
    assert e4m3.DECODE[0x38] == 1.0
    assert e4m3.DECODE[0xD0] == -8.0
    assert np.isnan(e4m3.DECODE[0x7F]) and np.isnan(e4m3.DECODE[0xFF])
    # every integer -16..16 is exact (the weight-side code property)
    for v in range(-16, 17):
        assert v in set(e4m3.DECODE[np.isfinite(e4m3.DECODE)].tolist())
    # codes 0x00..0x0F are exactly k * 2^-9 (subnormals, then the first normal binade)
    assert np.array_equal(e4m3.DECODE[:16], np.arange(16) * 2.0 ** -9)


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    d = e4m3.DECODE
    fin = np.isfinite(d)
    assert np.array_equal(np.isnan(t), ~fin)
    assert np.array_equal(t[fin], d[fin])


def test_spot_golden():
    rows = _spot_rows()
    assert len(rows) >= 15
    vals = np.array([v for v, _ in rows], dtype=np.float32)
    want = np.array([c for _, c in rows], dtype=np.uint8)
    got = e4m3.encode(vals)
    bad = [(float(v), hex(w), hex(g)) for v, w, g in zip(vals, want, got) if w != g]
    assert not bad, bad


def test_roundtrip_all_codes():
    """E(D(c)) == c for the 253 finite codes other than 0x80; 0x80 (-0) -> 0x00."""
    for c in range(256):
        if c in e4m3.NAN_CODES:
            continue
        v = np.float32(e4m3.DECODE[c])
        if c == 0x80:
            v = np.float32(-0.0)
            assert e4m3.encode(np.array([v]))[0] == 0x00
            continue
        assert e4m3.encode(np.array([v]))[0] == c, hex(c)


def test_specials():
    f = np.float32
    got = e4m3.encode(np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0], dtype=np.float32))
    assert got.tolist() == [0x00, 0x00, 0x7E, 0xFE, 0x00, 0x00]
    assert e4m3.encode(np.array([f(1e30)]))[0] == 0x7E


def _round_nearest_even_bruteforce(a):
    """Exhaustive nearest-value search over the table with exact rationals; ties -> even."""
    a = Fraction(float(a))
    a = min(a, Fraction(448))
    best = None
    for c in range(0x7F):
        d = abs(Fraction(float(e4m3.DECODE[c])) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_optimality_near_every_boundary():
    """Around each midpoint between neighbouring magnitudes (+-3 fp32 ulps) and at each
    representable value, the code is the exact-rational nearest, ties to even."""
    mags = e4m3.DECODE[:0x7F]
    pts = []
    for k in range(len(mags) - 1):
        mid = np.float32((mags[k] + mags[k + 1]) / 2)
        x = mid
        for _ in range(3):
            x = np.nextafter(x, np.float32(0))
        for _ in range(7):
            pts.append(x)
            x = np.nextafter(x, np.float32(np.inf))
    pts += [np.float32(m) for m in mags]
    pts = np.array(pts, dtype=np.float32)
    got = e4m3.encode(pts)
    for v, g in zip(pts, got):
        assert g == _round_nearest_even_bruteforce(v), (float(v), hex(g))
        assert e4m3.encode(np.array([-v]))[0] == (g | 0x80 if v != 0 else 0x00)


def test_against_torch_random_bitpatterns():
    """torch's float8_e4m3fn conversion is round-to-nearest-even; it agrees with E on every
    finite |q| <= 448 except that torch keeps the sign of -0.0."""
    r = np.random.default_rng(1234)
    bits = r.integers(0, 2 ** 32, 2 ** 22, dtype=np.uint64).astype(np.uint32)
    q = bits.view(np.float32)
    q = q[np.isfinite(q) & (np.abs(q) <= 448)]
    # also dense coverage of the small range where subnormal codes live
    q = np.concatenate([q, r.uniform(-0.05, 0.05, 2 ** 20).astype(np.float32)])
    ours = e4m3.encode(q)
    theirs = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    negzero = (q == 0) & np.signbit(q)
    assert np.array_equal(ours[~negzero], theirs[~negzero])
    assert np.all(ours[negzero] == 0)


@pytest.mark.parametrize("scale", [1.0, 1e-3, 100.0])
def test_monotone_and_symmetric(scale):
    x = np.sort(np.random.default_rng(7).uniform(0, 500 * scale, 100000).astype(np.float32))
    c = e4m3.encode(x).astype(np.int64)
    assert np.all(np.diff(c) >= 0)
    assert np.array_equal(e4m3.encode(-x[x > 0]) & 0x7F, c[x > 0] & 0x7F)
