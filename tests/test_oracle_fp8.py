"""Pins of the FP8 (E4M3, per-tensor) W8A8 oracle.

No GPU.  Each check uses something other than the oracle itself: torch's own
float8_e4m3fn conversion, exact rational arithmetic over every finite code,
representable inputs that must survive a round trip, the format's error bound,
and one-hot operands that expose a transposed or mis-scaled GEMM.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8 as P
from oracle.formats import e4m3_decode


def _torch_e4m3(y):
    """torch's float32 -> float8_e4m3fn cast (round to nearest even), as bytes."""
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    # wide dynamic range: normals, subnormals (below 2^-6), the top binade, exact ties
    y = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.uniform(-14, 8.8, 20000)),
        (np.arange(-4096, 4097) * 2.0 ** -12),                        # dense near zero, many ties
        e4m3_decode(np.arange(0x7F)) * rng.choice([-1, 1], 0x7F),     # every value itself
        np.array([448.0, -448.0, 432.0, 440.0, -0.0, 0.0, 2.0 ** -10, 3 * 2.0 ** -10]),
    ]).astype(np.float32)
    y = y[np.abs(y) <= 448.0]
    got = P.encode(y, np.float32(1.0))
    np.testing.assert_array_equal(got, _torch_e4m3(y))


def test_encode_brute_force_exact_nearest_signed():
    """Nearest of all 252 finite non-NaN signed codes in exact rationals, ties to the even code."""
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = {c: Fraction(float(e4m3_decode(c))) for c in codes}
    rng = np.random.default_rng(1)
    g = np.float32(0.0371)
    x = (rng.standard_normal(600) * 6.0).astype(np.float32)
    x[:3] = [0.0, -0.0, float(np.float32(448.0) * g)]
    got = P.encode(x, g)
    r = np.float32(np.float32(1.0) / g)
    for xi, gi in zip(x, got):
        y = Fraction(float(np.float32(xi * r)))
        y = max(min(y, Fraction(448)), Fraction(-448))
        best = min(abs(y - v) for v in vals.values())
        cands = [c for c, v in vals.items() if abs(y - v) == best]
        if len(cands) > 1:  # a tie (or +-0): even code, sign of x
            cands = [c for c in cands if (c & 1) == 0]
            cands = [c for c in cands if (c >> 7) == int(np.signbit(xi))] or cands
        assert len(cands) == 1 or all(vals[c] == 0 for c in cands)
        want = cands[0] if len(cands) == 1 else (0x80 if np.signbit(xi) else 0x00)
        assert gi == want, (xi, gi, want)


def test_dynamic_scale_and_amax_code():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 96)) * 3.0).astype(np.float32)
    q, g = P.quantize(x)
    assert g == np.float32(np.abs(x).max() / np.float32(448.0))
    i = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert q[i] == (0xFE if x[i] < 0 else 0x7E)  # the largest element lands on +-448
    assert np.all((q & 0x7F) != 0x7F)            # never the NaN code
    # sign symmetry: negating the input flips exactly the sign bit
    q2, g2 = P.quantize(-x)
    assert g2 == g
    np.testing.assert_array_equal(q2, q ^ 0x80)


def test_representable_round_trip():
    rng = np.random.default_rng(3)
    g = np.float32(2.0 ** -5)
    codes = rng.integers(0, 0x7F, 4096).astype(np.uint8) | (rng.integers(0, 2, 4096) << 7).astype(np.uint8)
    codes[0] = 0x7E  # holds the amax, so the dynamic scale is exactly g
    x = (e4m3_decode(codes) * np.float64(g)).astype(np.float32).reshape(64, 64)
    q, gq = P.quantize(x)
    assert gq == g
    np.testing.assert_array_equal(P.dequantize(q, gq), x.astype(np.float64))
    # codes come back except that -0 and +0 both mean zero
    same = (q == codes.reshape(64, 64)) | ((q & 0x7F) == 0) & ((codes.reshape(64, 64) & 0x7F) == 0)
    assert same.all()


def test_error_bound():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((32, 512)) * np.exp(rng.standard_normal(512))).astype(np.float32)
    q, g = P.quantize(x)
    err = np.abs(P.dequantize(q, g) - x.astype(np.float64))
    a = np.abs(x.astype(np.float64)) / np.float64(g)
    # half a code gap: 2^(e-4) for normals (3 mantissa bits), 2^-10 below 2^-6, in units of g
    half_gap = np.where(a < 2.0 ** -6, 2.0 ** -10, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4))
    assert np.all(err <= half_gap * np.float64(g) * (1 + 1e-5) + 1e-30)


def test_static_scale_saturates_and_zero_tensor():
    x = np.array([[1.0, -2.0, 0.25, 1e-6, -0.0, 0.0, 300.0, -5.0]], dtype=np.float32)
    q, g = P.quantize(x, g=np.float32(2.0 ** -3))  # 1/g = 8: 300*8 = 2400 > 448
    assert q[0, 6] == 0x7E and q[0, 1] == 0x80 | 0x58  # -16 = -(1+0)*2^4: e=11 -> 0x58
    assert q[0, 0] == 0x50 and q[0, 7] == 0xE2       # 8 = 2^3 (e=10); -40 = -1.25*2^5 (e=12, m=2)
    assert q[0, 4] == 0x80 and q[0, 5] == 0x00
    z, gz = P.quantize(np.zeros((4, 32), np.float32))
    assert gz == np.float32(1.0) and not z.any()
    with pytest.raises(ValueError):
        P.quantize(x, g=np.float32(0.0))
    with pytest.raises(ValueError):
        P.quantize(np.array([np.inf], np.float32))


def test_gemm_exact_small_and_one_hot_columns():
    rng = np.random.default_rng(5)
    M, N, K = 5, 7, 48
    a_q = rng.integers(0, 256, (M, K)).astype(np.uint8)
    b_q = rng.integers(0, 256, (N, K)).astype(np.uint8)
    a_q[(a_q & 0x7F) == 0x7F] = 0x38
    b_q[(b_q & 0x7F) == 0x7F] = 0xB8
    a_g, b_g = np.float32(0.125), np.float32(3.0)
    y = P.gemm(a_q, a_g, b_q, b_g)
    for i in range(M):
        for j in range(N):
            ref = sum(Fraction(float(e4m3_decode(a_q[i, k]))) * Fraction(float(e4m3_decode(b_q[j, k])))
                      for k in range(K)) * Fraction(0.125) * Fraction(3.0)
            assert abs(Fraction(float(y[i, j])) - ref) <= abs(ref) * Fraction(1, 2 ** 48)
    # one-hot A (code 0x38 = 1.0 at column k_i) picks column k_i of B, times both scales
    k_of = [3, 0, 47, 12, 12]
    a1 = np.zeros((M, K), np.uint8)
    a1[np.arange(M), k_of] = 0x38
    y1 = P.gemm(a1, np.float32(2.0), b_q, b_g)
    np.testing.assert_array_equal(y1, (e4m3_decode(b_q[:, k_of]).T * 2.0 * 3.0))
    sub = P.gemm_rows(a_q, a_g, b_q, b_g, [4, 1], [6, 0])
    np.testing.assert_array_equal(sub, y[[4, 1]][:, [6, 0]])
    with pytest.raises(ValueError):
        P.gemm(a_q, a_g, b_q[:, :16], b_g)
