"""Pins for oracle.formats against the pages, the format definitions and exact arithmetic.

No GPU.  Each check uses something other than the oracle itself: hand-written
tables from the pages' format names, exact rational arithmetic, an independent
bit-level rounding routine, or torch's float8_e4m3fn conversion.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def _f32_neighbours(v, n=8):
    """float32 values within n ulps of v (both sides), v itself included."""
    v = np.float32(v)
    out = [v]
    up = dn = v
    for _ in range(n):
        up = np.nextafter(up, np.float32(np.inf), dtype=np.float32)
        dn = np.nextafter(dn, np.float32(-np.inf), dtype=np.float32)
        out += [up, dn]
    return out


# ------------------------------------------------------------------ E2M1


def test_e2m1_decode_matches_hand_table(golden):
    rows = [r.split() for r in golden("e2m1_codes.txt")]
    codes = np.array([int(c) for c, _ in rows])
    want = np.array([float(v) for _, v in rows])
    got = F.e2m1_decode(codes)
    np.testing.assert_array_equal(got, want)
    # signs, including the negative zero of code 8
    np.testing.assert_array_equal(np.signbit(got), np.signbit(want))


def test_e2m1_grid_is_the_eight_value_grid():
    assert list(F.E2M1_MAGNITUDES) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert F.E2M1_MAX == 6.0


def test_e2m1_ties_match_hand_table(golden):
    for row in golden("e2m1_ties.txt"):
        mid, lo, hi, want = row.split()
        mid = float(mid)
        assert F.E2M1_MAGNITUDES[int(lo)] < mid < F.E2M1_MAGNITUDES[int(hi)]
        assert int(F.e2m1_encode(np.float32(mid))) == int(want)
        assert int(F.e2m1_encode(np.float32(-mid))) == int(want) | 8


def _exact_nearest_e2m1(y):
    """Brute force over the 8 magnitudes in exact rationals, ties to even code."""
    a = min(abs(Fraction(float(y))), Fraction(6))
    best, best_d = None, None
    for c in range(8):
        d = abs(a - Fraction(float(F.E2M1_MAGNITUDES[c])))
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (8 if np.signbit(y) else 0)


def _e2m1_points():
    pts = []
    for g in list(F.E2M1_MAGNITUDES) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0, 1e6]:
        for s in (1.0, -1.0):
            pts += _f32_neighbours(np.float32(g * s), n=6)
    rng = np.random.default_rng(123)
    pts += list(rng.uniform(-7.0, 7.0, 4000).astype(np.float32))
    pts += [np.float32(1e-30), np.float32(-1e-30), np.float32(-0.0), np.float32(0.0),
            np.float32(1.4e-45), np.float32(3.4e38), np.float32(-3.4e38)]
    return np.array(pts, dtype=np.float32)


def test_e2m1_encode_equals_exact_brute_force():
    pts = _e2m1_points()
    got = F.e2m1_encode(pts)
    want = np.array([_exact_nearest_e2m1(y) for y in pts], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(pts[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def _bitwise_e2m1(y):
    """Independent route: float32 bit-level round-to-nearest-even of |y| to the E2M1 grid.

    Below 1 the grid is uniform with step 0.5 (code = RNE(2|y|)); from 1 up it is a
    float with one mantissa bit, so rounding the float32 mantissa to 1 bit (RNE)
    and rebasing the exponent gives the code directly.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y), np.float32(6.0))
    small = np.rint(a.astype(np.float64) * 2).astype(np.int64)  # 2a is exact
    bits = a.view(np.uint32).astype(np.int64)
    rounded = (bits + 0x1FFFFF + ((bits >> 22) & 1)) >> 22
    big = rounded - (126 << 1)
    mag = np.where(a < 1.0, small, big)
    return (mag | (np.signbit(y).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_encode_equals_bitwise_rounding():
    rng = np.random.default_rng(7)
    pts = np.concatenate([_e2m1_points(),
                          rng.standard_normal(200000).astype(np.float32) * 3,
                          rng.uniform(-6.5, 6.5, 200000).astype(np.float32)])
    np.testing.assert_array_equal(F.e2m1_encode(pts), _bitwise_e2m1(pts))


def test_e2m1_rejects_non_finite():
    with pytest.raises(ValueError):
        F.e2m1_encode(np.array([np.inf], dtype=np.float32))


# ------------------------------------------------------------------ E4M3


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_format_constants_match_the_page(golden):
    """The audit's largest scale, 448.0, is E4M3FN's largest finite value."""
    audit = dict(r.split(": ") for r in golden("scale_audit.txt"))
    assert float(audit["scale_max"]) == F.E4M3_MAX == np.nanmax(F.e4m3_decode(np.arange(256)))
    assert F.E4M3_MIN_POS == F.e4m3_decode(1) == 2.0 ** -9
    recipe = dict(r.split(": ") for r in golden("nvfp4_recipe.txt"))
    # scale_bits [4,3]: 4 exponent + 3 mantissa bits + sign = one byte per scale
    assert int(recipe["scale_bits_exponent"]) + int(recipe["scale_bits_mantissa"]) + 1 == 8
    assert len(F.E4M3_NONNEG) == 127 and np.all(np.diff(F.E4M3_NONNEG) > 0)


def _e4m3_points():
    pts = []
    for v in F.E4M3_NONNEG:
        pts += _f32_neighbours(v, n=4)
    mids = (F.E4M3_NONNEG[1:] + F.E4M3_NONNEG[:-1]) / 2
    for v in mids:
        pts += _f32_neighbours(v, n=4)
    rng = np.random.default_rng(5)
    pts += list(np.exp(rng.uniform(np.log(1e-6), np.log(448.0), 20000)).astype(np.float32))
    pts = np.array(pts, dtype=np.float32)
    return pts[(pts >= 0) & (pts <= 448.0)]


def test_e4m3_encode_matches_torch_cast():
    pts = _e4m3_points()
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(pts)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(pts[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_encode_equals_exact_brute_force_small_sample():
    pts = _e4m3_points()[::7]
    table = [Fraction(float(v)) for v in F.E4M3_NONNEG]
    got = F.e4m3_encode(pts)
    for v, c in zip(pts, got):
        fv = Fraction(float(v))
        dists = [abs(fv - t) for t in table]
        dmin = min(dists)
        cands = [i for i, d in enumerate(dists) if d == dmin]
        want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        assert int(c) == want, (float(v), int(c), want)


def test_e4m3_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([449.0], dtype=np.float32))
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([-1.0], dtype=np.float32))
