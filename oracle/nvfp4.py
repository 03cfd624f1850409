"""Two-level NVFP4 quantize and dequantize.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (two-level scaling page, section "Core: the W4A4 two-level
scaling mechanism"):

* level 1 -- the tensor is cut into 16-element blocks along its last dimension;
  each block shares one E4M3 scale and each element is a 4-bit E2M1 code;
* level 2 -- one FP32 global scale per tensor moves the whole distribution into
  the range FP4 represents;
* every scale is finite and positive, the largest is 448.0 (scale audit);
* 4.5 bits per element (sub-section "Why 4.5 bits");
* activations use the same 16-block rule, computed on the fly (sub-section
  "The A4 side: dynamic activations"); weights are quantized offline.

What the pages leave open, and the reading taken (all float32 IEEE arithmetic,
round-to-nearest-even, denormals kept; ``fl`` = one rounding):

1. ``amax = max |x|`` over the whole tensor.
2. Stored global scale is the *decode* multiplier ``g = fl(amax / 2688)``
   (2688 = 6 * 448, the largest E2M1 value times the largest E4M3 value), or
   ``g = 1`` for an all-zero tensor.  This puts the block holding ``amax`` at
   block scale 448, matching the audit's maximum; the audit's smallest value
   (about 2e-5) is the size of ``g`` for weights of spread 0.02.
3. Per block ``bmax = max |x|`` and ``s32 = fl(bmax / fl(6 * g))``.
4. ``s = E4M3_RNE(min(s32, 448))``; a scale that rounds to zero becomes the
   smallest positive E4M3 value 2**-9 (scales are positive per the audit).
5. ``r = fl(1 / fl(s * g))``, one reciprocal per block.
6. ``y = fl(x * r)`` and ``code = E2M1_RNE(min(|y|, 6))`` with the sign of ``x``.
7. Codes packed two per byte, even element in the low nibble; scales stored one
   byte per block, row-major.
8. Dequantize: ``x_hat = e2m1(code) * e4m3(s) * g``, exact in float64.

Preconditions: finite input; ``amax`` is 0 or at least 2**-100 (so that ``r``
stays finite).  With a caller-supplied ("static") global scale, ``g`` must be a
positive normal float32 of at least 2**-100.
"""

import numpy as np

from .formats import e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode

BLOCK = 16
#: 6 (E2M1 max) * 448 (E4M3 max)
GLOBAL_DIVISOR = np.float32(2688.0)
#: smallest non-zero amax (and smallest static global scale) accepted
MIN_AMAX = 2.0 ** -100


def global_scale(x):
    """Step 1-2: the per-tensor FP32 decode scale of float32 tensor ``x``."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    if amax < MIN_AMAX:
        raise ValueError("quantize: amax below the supported minimum 2**-100")
    return np.float32(amax / GLOBAL_DIVISOR)


def block_scales(x, g):
    """Steps 3-4: E4M3 code of every 16-element block of float32 ``x`` [rows, cols]."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    g = np.float32(g)
    bmax = np.abs(x).reshape(rows, cols // BLOCK, BLOCK).max(axis=-1)
    six_g = np.float32(np.float32(6.0) * g)
    s32 = (bmax / six_g).astype(np.float32)
    s = e4m3_encode(np.minimum(s32, np.float32(448.0)))
    s[s == 0] = 1
    return s


def encode_elements(x, s, g):
    """Steps 5-6: E2M1 codes of float32 ``x`` [rows, cols] given block scale codes."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    g = np.float32(g)
    s_val = e4m3_decode(s).astype(np.float32)
    r = (np.float32(1.0) / (s_val * g).astype(np.float32)).astype(np.float32)
    y = (x.reshape(rows, cols // BLOCK, BLOCK) * r[..., None]).astype(np.float32)
    return e2m1_encode(y).reshape(rows, cols)


def pack_codes(codes):
    """Step 7: two 4-bit codes per byte, element 2j in bits 3..0, 2j+1 in bits 7..4."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(q):
    """Inverse of :func:`pack_codes`."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def quantize(x, g=None):
    """Quantize a 2-D float32 tensor (bf16 callers widen exactly first).

    Returns ``(q, s, g)``: packed codes uint8 [rows, cols/2], block scale codes
    uint8 [rows, cols/16], global scale float32.  ``g=None`` is the dynamic
    (activation) mode; a given ``g`` is the static mode.
    """
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
    s = block_scales(x, g)
    codes = encode_elements(x, s, g)
    return pack_codes(codes), s, np.float32(g)


def dequantize(q, s, g):
    """Step 8: exact float64 value of every element."""
    codes = unpack_codes(q)
    rows, cols = codes.shape
    sv = e4m3_decode(s).astype(np.float64)
    vals = e2m1_decode(codes).reshape(rows, cols // BLOCK, BLOCK) * sv[..., None]
    return vals.reshape(rows, cols) * np.float64(g)


def effective_bits(q, s, numel):
    """Storage bits per element of the per-element payload (codes + block scales)."""
    return (np.asarray(q).nbytes + np.asarray(s).nbytes) * 8 / numel
