"""Quantize-dequantize ("fake quantization"): the forward of quantization-aware
training.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages say: Model-Optimizer simulates NVFP4 during PTQ calibration and
QAD by quantizing and immediately dequantizing in the forward pass, so the
model sees the values NVFP4 can hold while staying in a wide format (QAD page,
sections on the QAD workflow and on scale handling: dynamic scales recomputed
every step, or frozen calibrated ones).

Reading taken: ``y = fl_out(fl32(e2m1(code) * e4m3(s) * g))`` for the codes and
scales of the plain quantizer (``nvfp4``), dynamic or static ("frozen") global
scale; ``e2m1 * e4m3`` is exact, the product with ``g`` is rounded once to
float32, and a bfloat16 output rounds that float32 once more, to nearest even.
"""

import numpy as np

from .nvfp4 import dequantize, quantize


def round_to_bf16(x):
    """float32 -> the nearest bfloat16 (ties to even), returned as float32 values."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def qdq(x, g=None, out="f32"):
    """Fake-quantize a 2-D float32 tensor -> (y float32 values, g)."""
    q, s, g = quantize(x, g=g)
    y = dequantize(q, s, g).astype(np.float32)  # exact product, one rounding
    if out == "bf16":
        y = round_to_bf16(y)
    elif out != "f32":
        raise ValueError("out must be 'f32' or 'bf16'")
    return y, g
