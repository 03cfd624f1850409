"""The W4A4 NVFP4 GEMM as an exact-operand float64 product.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Model-Optimizer QAD tutorial for Qwen3.6-35B-A3B, section "Why W4A4 rather than
W4A16": both the weight and the activation operand are 4-bit NVFP4, so the
product runs on FP4 units with a wide accumulator; the two-level scaling page
(section "Core: the W4A4 two-level scaling mechanism") fixes what each operand
means: ``value = e2m1(code) * e4m3(block scale) * global scale``.

The GEMM therefore has a plain definition: ``Y = A_hat @ B_hat^T`` where ``A`` is
[M, K] and ``B`` is [N, K], both quantized along K (their last dimension), and
``*_hat`` are the exactly dequantized operands.  It is evaluated in float64 by
numpy's matmul; every dequantized value is exact in float64, so the only error
is float64 summation rounding (relative ~K * 2**-53), far below any tolerance.
"""

import numpy as np

from .nvfp4 import dequantize


def gemm(a_q, a_s, a_g, b_q, b_s, b_g):
    """Y[M, N] (float64) = dequant(A) @ dequant(B)^T."""
    a = dequantize(a_q, a_s, a_g)
    b = dequantize(b_q, b_s, b_g)
    if a.shape[1] != b.shape[1]:
        raise ValueError("gemm: K mismatch")
    return a @ b.T


def gemm_rows(a_q, a_s, a_g, b_q, b_s, b_g, rows, cols=None):
    """Selected outputs Y[rows][:, cols] without forming the whole product."""
    a = dequantize(np.asarray(a_q)[rows], np.asarray(a_s)[rows], a_g)
    if cols is None:
        b = dequantize(b_q, b_s, b_g)
    else:
        b = dequantize(np.asarray(b_q)[cols], np.asarray(b_s)[cols], b_g)
    return a @ b.T


def rel_fro_error(y, y_ref):
    """||y - y_ref||_F / ||y_ref||_F in float64."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    return float(num / den) if den > 0 else float(num)
