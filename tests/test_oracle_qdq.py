"""Pins of the quantize-dequantize oracle: bfloat16 rounding, representable
inputs, idempotence with a frozen scale, and the error bound."""

import numpy as np
import pytest
import torch

from oracle import nvfp4 as Q
from oracle import qdq as D
from oracle.formats import E2M1_MAGNITUDES


def test_bf16_rounding_matches_torch_and_ties_to_even():
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, 3.14159, -2.7182817, 1e-30, 65504.0,
                     1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).float().numpy()
    assert np.array_equal(D.round_to_bf16(vals), ref)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even 1.0
    assert D.round_to_bf16(np.float32(1.0 + 2 ** -8)) == np.float32(1.0)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6
    assert D.round_to_bf16(np.float32(1.0 + 3 * 2 ** -8)) == np.float32(1.0 + 2 ** -6)


def test_representable_inputs_pass_through():
    # every value e2m1 * 2^-4 with the tensor max 6 * 2^-4: g = 6*2^-4/2688, block scale
    # 448 only in the max block; use blocks whose max is 6 * 2^k with s = 2^k / g exact
    g = np.float32(2.0 ** -8)
    s_vals = [1.0, 8.0, 64.0, 0.5]
    rng = np.random.default_rng(0)
    rows = []
    for sv in s_vals:
        mags = rng.choice(E2M1_MAGNITUDES, 15)
        blk = np.concatenate([[6.0], mags]) * sv * np.float64(g)
        rows.append(blk * rng.choice([-1, 1], 16))
    x = np.array(rows, dtype=np.float32).reshape(1, -1)
    y, _ = D.qdq(x, g=g)
    assert np.array_equal(y, x)


def test_idempotent_with_frozen_scale():
    x = (np.random.default_rng(1).standard_normal((8, 256)) * 0.5).astype(np.float32)
    g = Q.global_scale(x)
    y1, _ = D.qdq(x, g=g)
    y2, _ = D.qdq(y1, g=g)
    assert np.array_equal(y1, y2)


def test_error_bound_and_dynamic_scale():
    x = (np.random.default_rng(2).standard_normal((16, 512)) * np.exp(np.random.default_rng(3)
                                                                      .standard_normal(512))).astype(np.float32)
    y, g = D.qdq(x)
    assert g == Q.global_scale(x)
    q, s, _ = Q.quantize(x)
    step = 2.0 * Q.e4m3_decode(s).astype(np.float64) * np.float64(g)  # largest E2M1 gap is 2
    err = np.abs(y.astype(np.float64) - x).reshape(16, -1, 16).max(-1)
    assert np.all(err <= step / 2 * (1 + 1e-6))
    yb, _ = D.qdq(x, out="bf16")
    assert np.array_equal(yb, D.round_to_bf16(y))
    with pytest.raises(ValueError):
        D.qdq(x, out="f16")
