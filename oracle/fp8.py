"""FP8 (E4M3) W8A8 per-tensor linear layer: quantize, dequantize, GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

* QAD tutorial, section on the quantized checkpoint's contents (the table of
  quantized tensors by module): the linear-attention and full-attention
  projections of the W4A4 checkpoint stay in FP8 W8A8, next to the NVFP4 MoE
  experts.
* Format-selection guide, section 1 (the format table): FP8 is W8A8 with
  per-tensor scaling, half the weight memory.
* Two-level scaling page, section "Core: the W4A4 two-level scaling mechanism":
  the FP8 of this model family is E4M3 (``F8_E4M3``) with a scalar FP32 scale
  per tensor that the reader must multiply back in; its largest value 448 makes
  it the E4M3FN variant (see ``formats``).

What the pages leave open, and the reading taken (float32 IEEE arithmetic,
round-to-nearest-even, denormals kept; ``fl`` = one rounding):

1. ``amax = max |x|`` over the whole tensor.
2. The stored per-tensor scale is the *decode* multiplier ``g = fl(amax / 448)``,
   so the largest element lands on the largest code; ``g = 1`` for an all-zero
   tensor.  A caller may also supply ``g`` (static scale, as calibrated
   checkpoints store it).
3. ``r = fl(1 / g)``, one reciprocal per tensor.
4. ``y = fl(x * r)`` and ``code = E4M3_RNE(min(|y|, 448))`` with the sign bit of
   ``x`` copied (so -0 and negatives that round to zero give 0x80).  The clamp
   makes a static scale below the data's range saturate at +-448 instead of
   producing the NaN code.
5. Dequantize: ``x_hat = e4m3(code) * g``, exact in float64.
6. GEMM: ``Y = A_hat @ B_hat^T`` with ``A`` [M, K] and ``B`` [N, K] (the weight
   stored row-major as [out, in]); every operand value is exact in float64, so
   the float64 product's only error is summation rounding (relative about
   K * 2**-53).

Preconditions: finite input; ``amax`` is 0 or at least 2**-100 (so that ``r``
stays finite); a static ``g`` is a float32 of at least 2**-100.
"""

import numpy as np

from .formats import E4M3_MAX, e4m3_decode, e4m3_encode

#: smallest non-zero amax (and smallest static scale) accepted
MIN_AMAX = 2.0 ** -100


def scale(x):
    """Steps 1-2: the per-tensor FP32 decode scale of float32 tensor ``x``."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    if amax < MIN_AMAX:
        raise ValueError("fp8 quantize: amax below the supported minimum 2**-100")
    return np.float32(amax / np.float32(E4M3_MAX))


def encode(x, g):
    """Steps 3-4: signed E4M3FN code (uint8) of every element of float32 ``x``."""
    x = np.asarray(x, dtype=np.float32)
    g = np.float32(g)
    r = np.float32(np.float32(1.0) / g)
    y = (x * r).astype(np.float32)
    mag = e4m3_encode(np.minimum(np.abs(y), np.float32(E4M3_MAX)))
    sign = np.signbit(x).astype(np.uint8)
    return ((sign << 7) | mag).astype(np.uint8)


def quantize(x, g=None):
    """Quantize a float32 tensor (bf16 callers widen exactly first).

    Returns ``(q, g)``: uint8 E4M3FN codes of ``x``'s shape and the float32
    decode scale.  ``g=None`` is the dynamic mode; a given ``g`` is static.
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("fp8 quantize: non-finite input")
    if g is None:
        g = scale(x)
    else:
        g = np.float32(g)
        if not (np.isfinite(g) and g >= MIN_AMAX):
            raise ValueError("fp8 quantize: static scale must be finite and >= 2**-100")
    return encode(x, g), np.float32(g)


def dequantize(q, g):
    """Step 5: exact float64 value of every code."""
    return e4m3_decode(q) * np.float64(g)


def gemm(a_q, a_g, b_q, b_g):
    """Step 6: Y[M, N] (float64) = dequant(A) @ dequant(B)^T."""
    a = dequantize(a_q, a_g)
    b = dequantize(b_q, b_g)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("fp8 gemm: need A [M, K] and B [N, K]")
    return a @ b.T


def gemm_rows(a_q, a_g, b_q, b_g, rows, cols=None):
    """Selected outputs Y[rows][:, cols] without forming the whole product."""
    a = dequantize(np.asarray(a_q)[rows], a_g)
    b = dequantize(b_q if cols is None else np.asarray(b_q)[cols], b_g)
    return a @ b.T
