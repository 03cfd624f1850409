"""E2M1 (FP4) and E4M3 (FP8) number formats, decode and round-to-nearest-even encode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Two-level scaling page, section "Core: the W4A4 two-level scaling mechanism":
elements are 4-bit E2M1 (recipe ``num_bits: [2, 1]``: 2 exponent bits, 1 mantissa
bit) and each 16-element block carries an FP8 E4M3 scale (recipe
``scale_bits: [4, 3]``: 4 exponent bits, 3 mantissa bits).  The scale audit on
that page reports a largest scale of exactly 448.0, the largest finite value of
the OCP "E4M3FN" variant (the FNUZ variant stops at 240), so E4M3 here is E4M3FN:
exponent bias 7, subnormals, no infinities, 0x7F/0xFF are NaN.

E2M1 layout: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.  Exponent
field 0 is subnormal (0 or 0.5); there are no infinities or NaNs.

Encoding is "nearest representable value, ties to the even code" (the even code
is the one whose mantissa LSB, i.e. code LSB, is 0), the usual IEEE
round-to-nearest-even restricted to the format's grid.  The pages do not name a
rounding mode; RNE is the reading taken.

Exactness of the nearest search: candidates are compared by |a - v| computed in
float64.  A tie can only happen when ``a`` sits exactly on a midpoint between two
grid values; a float32 ``a`` within a few binades of the grid values makes
``a - v`` exact in float64 (24 + at most 20 significant bits), and when ``a`` is
far from every midpoint the float64 rounding error (relative 2**-53) is far below
the gap between the two distances.  So the search decides exactly like exact
rational arithmetic would; tests/test_oracle_formats.py checks this against
exact fractions.
"""

import numpy as np

# --------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (float64).  Codes are taken modulo 16."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(sign == 1, -mag, mag)


#: magnitudes of the 8 non-negative codes 0..7, in code order
E2M1_MAGNITUDES = e2m1_decode(np.arange(8))
#: largest E2M1 magnitude
E2M1_MAX = 6.0


def _nearest_code(a, table):
    """Index into ``table`` (ascending, distinct) nearest to each ``a``.

    Ties between two neighbours go to the even index.  ``a`` is float64 holding
    float32 values.
    """
    a = np.asarray(a, dtype=np.float64)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    step = max(1, (1 << 22) // len(table))  # bounds the temporary distance matrix
    for lo in range(0, flat.size, step):
        chunk = flat[lo:lo + step]
        d = np.abs(chunk[:, None] - table)
        cand = d == d.min(axis=1, keepdims=True)
        first = np.argmax(cand, axis=1)
        last = cand.shape[1] - 1 - np.argmax(cand[:, ::-1], axis=1)
        out[lo:lo + step] = np.where(first % 2 == 0, first, last)
    return out.reshape(a.shape)


def e2m1_encode(y):
    """E2M1 code of float32 ``y``: nearest magnitude (ties to even), saturating at 6.

    The sign bit copies the sign of ``y``, including negative zero (reading: sign
    is kept, so -0.0 and small negatives that round to zero give code 0x8).
    Input must be finite.
    """
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("e2m1_encode: non-finite input")
    a = np.minimum(np.abs(y).astype(np.float64), E2M1_MAX)
    mag = _nearest_code(a, E2M1_MAGNITUDES).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8)
    return (sign << 3) | mag


# --------------------------------------------------------------------------
# E4M3 (E4M3FN)
# --------------------------------------------------------------------------


def e4m3_decode(codes):
    """Value of each 8-bit E4M3FN code (float64); 0x7F and 0xFF decode to NaN."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(sign == 1, -mag, mag)


#: the 127 non-negative finite E4M3FN values, codes 0x00..0x7E in code order
E4M3_NONNEG = e4m3_decode(np.arange(0x7F))
#: largest finite E4M3FN value
E4M3_MAX = 448.0
#: smallest positive E4M3FN value (subnormal, code 0x01)
E4M3_MIN_POS = 2.0 ** -9


def e4m3_encode(v):
    """E4M3FN code of a non-negative float32 ``v`` <= 448: nearest value, ties to even.

    Callers clamp to 448 first (the quantizer does); values above 448 raise.
    """
    v = np.asarray(v, dtype=np.float32)
    if np.any(~np.isfinite(v)) or np.any(v < 0) or np.any(v > E4M3_MAX):
        raise ValueError("e4m3_encode: input must be finite and in [0, 448]")
    return _nearest_code(v.astype(np.float64), E4M3_NONNEG).astype(np.uint8)
