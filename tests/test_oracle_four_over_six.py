"""Pins of the four-over-six oracle (block maxima mapped to 6 or to 4 by lower
squared error), against the plain quantizer, float64 errors and hand-built blocks."""

import numpy as np
import pytest

from oracle import four_over_six as F
from oracle import nvfp4 as Q
from oracle.formats import e2m1_decode


def _rand(rows, cols, seed, std=0.02):
    return (np.random.default_rng(seed).standard_normal((rows, cols)) * std).astype(np.float32)


def test_m6_candidate_is_the_plain_quantizer():
    x = _rand(32, 256, 1)
    g = Q.global_scale(x)
    s6 = F.candidate_scales(x, g, 6)
    assert np.array_equal(s6, Q.block_scales(x, g))
    assert np.array_equal(Q.encode_elements(x, s6, g), Q.unpack_codes(Q.quantize(x)[0]))


def test_choice_agrees_with_float64_errors():
    # the float32 error sums decide; wherever the exact (float64) errors of the
    # two candidates differ by more than float32 rounding can move a sum of 16
    # squares, the choice must be the exact comparison's
    x = _rand(64, 512, 2)
    q, s, g, took4 = F.quantize(x)
    rows, cols = x.shape

    def exact_err(m):
        sm = F.candidate_scales(x, g, m)
        c = Q.encode_elements(x, sm, g)
        xh = (e2m1_decode(c).astype(np.float64).reshape(rows, -1, 16)
              * Q.e4m3_decode(sm)[..., None] * np.float64(g))
        return ((x.reshape(rows, -1, 16).astype(np.float64) - xh) ** 2).sum(-1)
    e6, e4 = exact_err(6), exact_err(4)
    clear = np.abs(e6 - e4) > 1e-4 * np.maximum(e6, e4)
    assert clear.mean() > 0.9
    assert np.array_equal(took4[clear], (e4 < e6)[clear])
    assert 0.1 < took4.mean() < 0.9  # both choices occur on Gaussian weights


def test_never_worse_than_plain_and_lower_overall():
    x = _rand(64, 512, 3)
    q, s, g, _ = F.quantize(x)
    q6, s6, g6 = Q.quantize(x)
    assert g == g6
    err46 = ((Q.dequantize(q, s, g) - x) ** 2).reshape(64, -1, 16).sum(-1)
    err6 = ((Q.dequantize(q6, s6, g6) - x) ** 2).reshape(64, -1, 16).sum(-1)
    assert np.all(err46 <= err6 * (1 + 1e-5) + 1e-30)
    assert err46.sum() < 0.95 * err6.sum()


def _one_block_tensor(block, other_max):
    """[1, 32]: the block under test, then a block holding the tensor's amax."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :16] = block
    x[0, 16] = other_max
    return x


def test_block_on_the_four_grid_takes_four():
    # with g = 1/16 (amax 168 = 2688/16) the block max 4 maps to s = 4/(4g) = 16,
    # an E4M3 value, and every element lies on the E2M1 grid times s g = 1: exact
    blk = np.array([4, 3, 2, 1.5, 1, 0.5, 0, -4, -3, -2, -1.5, -1, -0.5, 0, 3, 2], dtype=np.float32)
    x = _one_block_tensor(blk, 168.0)
    q, s, g, took4 = F.quantize(x)
    assert g == np.float32(1 / 16)
    assert took4[0, 0] and not took4[0, 1]
    assert np.array_equal(Q.dequantize(q, s, g)[0, :16], blk)


def test_block_on_the_six_grid_keeps_six():
    blk = np.array([6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, -2, -1.5, -1, -0.5, 0], dtype=np.float32)
    x = _one_block_tensor(blk, 168.0)
    q, s, g, took4 = F.quantize(x)
    assert not took4[0, 0]
    assert np.array_equal(Q.dequantize(q, s, g)[0, :16], blk)


def test_ties_keep_six():
    # all-zero block: both candidates give zero error; the amax block: both
    # candidates clamp to scale 448 and coincide
    x = _one_block_tensor(np.zeros(16, dtype=np.float32), 100.0)
    q, s, g, took4 = F.quantize(x)
    assert not took4.any()
    assert s[0, 0] == 1 and s[0, 1] == 0x7E


def test_static_scale_and_rejects():
    x = _rand(4, 64, 5)
    g = Q.global_scale(x)
    assert np.array_equal(F.quantize(x, g=g)[0], F.quantize(x)[0])
    with pytest.raises(ValueError):
        F.quantize(np.zeros((2, 24), dtype=np.float32))
    with pytest.raises(ValueError):
        F.quantize(x, g=np.float32(0))
