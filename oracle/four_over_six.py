"""Four-over-six block-scale selection for offline (weight) quantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages say: the PTQ recipe table of the Nemotron 3.5 Lightning QAD
page lists a "4/6" calibration: for every block, the block maximum is mapped
either to the largest E2M1 magnitude M = 6 (the plain NVFP4 rule) or to M = 4,
whichever gives the lower mean squared quantization error (the table cites
arXiv 2512.02010); such searched scales are fixed once and kept frozen
afterwards (the same page, section on scale handling during QAD).

Readings taken (float32 throughout, one rounding per operation, round to
nearest even):

1. The global scale ``g`` is the plain one (dynamic ``amax / 2688``, or a
   caller's static value): the tensor's largest block maps to 448 either way,
   because ``amax / (4 g)`` exceeds 448 and is clamped.
2. Candidate M in {6, 4}: ``s_M = E4M3(min(fl(bmax / fl(M g)), 448))``, a zero
   raised to 2**-9; codes from ``r = fl(1 / fl(s_M g))`` exactly as the plain
   quantizer does (``nvfp4`` steps 5-6).
3. Block error ``E_M``: with ``v_i = e2m1(code_i) * e4m3(s_M)`` (exact) and
   ``d_i = fl(x_i - fl(v_i * g))``, ``E_M = (((d_0^2 + d_1^2) + d_2^2) + ...)``,
   each square and each addition rounded once, in element order.  (The mean
   differs from the sum by the constant 1/16, which cannot change the choice.)
4. The block takes M = 4 iff ``E_4 < E_6``; a tie keeps the plain M = 6.

The float32 order of step 3 decides an integer (the choice), so the GPU path
takes the same decision in the same precision and order; it has no pin beyond
this definition, but the tests check the choice against the float64 errors
wherever those differ by more than float32 rounding can move them.
"""

import numpy as np

from .formats import e2m1_decode, e4m3_decode, e4m3_encode
from .nvfp4 import BLOCK, encode_elements, global_scale, MIN_AMAX, pack_codes


def candidate_scales(x, g, m):
    """Step 2: E4M3 code of every block for the mapping of bmax to ``m`` (6 or 4)."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    bmax = np.abs(x).reshape(rows, cols // BLOCK, BLOCK).max(axis=-1)
    mg = np.float32(np.float32(m) * np.float32(g))
    s32 = (bmax / mg).astype(np.float32)
    s = e4m3_encode(np.minimum(s32, np.float32(448.0)))
    s[s == 0] = 1
    return s


def block_errors(x, codes, s, g):
    """Step 3: float32 sum of squared errors of every block, in element order."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    g = np.float32(g)
    v = (e2m1_decode(codes).reshape(rows, cols // BLOCK, BLOCK)
         * e4m3_decode(s)[..., None]).astype(np.float32)  # exact products
    xh = (v * g).astype(np.float32)
    d = (x.reshape(rows, cols // BLOCK, BLOCK) - xh).astype(np.float32)
    e = np.zeros((rows, cols // BLOCK), dtype=np.float32)
    for i in range(BLOCK):
        sq = (d[..., i] * d[..., i]).astype(np.float32)
        e = (e + sq).astype(np.float32)
    return e


def quantize(x, g=None):
    """Four-over-six quantize of a 2-D float32 tensor -> ``(q, s, g, took4)``.

    ``took4`` is the boolean [rows, cols/16] choice of M = 4 (for tests)."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("quantize: need a 2-D tensor whose last dim is a multiple of 16")
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize: non-finite input")
    if g is None:
        g = global_scale(x)
    else:
        g = np.float32(g)
        if not (np.isfinite(g) and g >= MIN_AMAX):
            raise ValueError("quantize: static global scale must be finite and >= 2**-100")
    s6 = candidate_scales(x, g, 6)
    s4 = candidate_scales(x, g, 4)
    c6 = encode_elements(x, s6, g)
    c4 = encode_elements(x, s4, g)
    e6 = block_errors(x, c6, s6, g)
    e4 = block_errors(x, c4, s4, g)
    took4 = e4 < e6
    rows, cols = x.shape
    codes = np.where(np.repeat(took4, BLOCK, axis=1), c4, c6)
    s = np.where(took4, s4, s6).astype(np.uint8)
    return pack_codes(codes), s, np.float32(g), took4
