"""Routed-expert MoE layer with NVFP4 W4A4 experts.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

* two-level scaling page, section "Why only routed experts": each token is routed
  to k of E experts (top-10 of 512 there); the router stays in BF16 and picks the
  experts; only the routed experts' weights are NVFP4;
* same page, section "Step 1: what NVFP4 touched": each expert's projections are
  stored fused as ``gate_up_proj`` and ``down_proj``;
* same page, sub-section "The A4 side: dynamic activations": activations entering
  a quantized linear are quantized on the fly with the 16-block rule.

Readings taken where the pages are silent:

* top-k: logits sorted descending, equal logits ordered by lower expert id;
  slot j holds the j-th largest;
* routing weights: softmax over the k selected logits (equal to a full softmax
  followed by renormalisation over the selected k), float64;
* permutation: routed rows ordered by (expert, token, slot); a token picks
  distinct experts, so within an expert rows are in ascending token order;
* ``gate_up_proj`` is [2I, H]; rows [0, I) are the gate, rows [I, 2I) the up
  projection; ``h = SiLU(gate) * up`` with ``SiLU(z) = z / (1 + exp(-z))``;
* one global scale per quantize call: the token activations X before
  permutation (one tensor), h over all routed rows (one tensor), and each expert's
  gate_up and down matrices (one tensor each);
* the combine sums ``w[t, j] * y[row(t, j)]`` over slots j = 0..k-1 in order;
* the intermediates h and y are stored either as float32 or, as serving engines
  keep activations, in bfloat16 (rounded to nearest even from float32); the
  quantizer of h reads the stored h and the combine the stored y.
"""

import numpy as np

from .nvfp4 import quantize, dequantize
from .qdq import round_to_bf16


def topk(logits, k):
    """(ids int32 [T, k], selected logits float32 [T, k]) of float32 router logits."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("topk: need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # stable sort on the negated logits keeps lower ids first among equals
        order = np.argsort(-logits[t], kind="stable")
        ids[t] = order[:k]
    return ids, np.take_along_axis(logits, ids.astype(np.int64), axis=1)


def softmax_weights(sel_logits):
    """Softmax over the k selected logits of each token, float64."""
    z = np.asarray(sel_logits, dtype=np.float64)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def route(logits, k):
    """(topk_ids int32 [T, k], topk_w float64 [T, k])."""
    ids, sel = topk(logits, k)
    return ids, softmax_weights(sel)


def permute(topk_ids, num_experts):
    """Group the T*k routed (token, slot) pairs by expert.

    Returns ``offsets`` int32 [E+1] (rows of expert e are offsets[e]:offsets[e+1]),
    ``src_row`` int32 [R] (token of each routed row) and ``inv`` int32 [T, k]
    (routed row of each (token, slot)).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    pairs = [(int(ids[t, j]), t, j) for t in range(T) for j in range(k)]
    pairs.sort()
    counts = np.bincount(ids.reshape(-1), minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    src_row = np.array([t for (_, t, _) in pairs], dtype=np.int32)
    inv = np.empty((T, k), dtype=np.int32)
    for r, (_, t, j) in enumerate(pairs):
        inv[t, j] = r
    return offsets, src_row, inv


def silu_gate(gu):
    """h = SiLU(gate) * up for gate_up outputs [R, 2I] (gate first), float64."""
    gu = np.asarray(gu, dtype=np.float64)
    i = gu.shape[1] // 2
    gate, up = gu[:, :i], gu[:, i:]
    return gate / (1.0 + np.exp(-gate)) * up


def grouped_gemm(a_q, a_s, a_g, src_row, offsets, w_q, w_s, w_g):
    """Per expert e: rows offsets[e]:offsets[e+1] of the gathered A times W_e^T.

    ``a_*`` is the quantized source tensor; routed row r reads source row
    ``src_row[r]`` (``src_row=None`` means row r).  ``w_q/w_s/w_g`` are per-expert
    stacks [E, N, K/2], [E, N, K/16], [E].  Returns float64 [R, N].
    """
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    R = int(offsets[-1])
    N = np.asarray(w_q).shape[1]
    out = np.zeros((R, N), dtype=np.float64)
    idx = np.arange(R) if src_row is None else np.asarray(src_row)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = idx[lo:hi]
        a = dequantize(np.asarray(a_q)[rows], np.asarray(a_s)[rows], a_g)
        w = dequantize(w_q[e], w_s[e], w_g[e])
        out[lo:hi] = a @ w.T
    return out


def combine(y, topk_w, inv):
    """out[t] = sum_j w[t, j] * y[inv[t, j]], slots in order, float64 [T, H]."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(topk_w, dtype=np.float64)
    inv = np.asarray(inv)
    T, k = inv.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[inv[:, j]]
    return out


def quantize_experts(w):
    """Quantize a stack of expert matrices [E, N, K] (float32), one global scale each."""
    w = np.asarray(w, dtype=np.float32)
    qs, ss, gs = zip(*(quantize(w[e]) for e in range(w.shape[0])))
    return np.stack(qs), np.stack(ss), np.array(gs, dtype=np.float32)


def moe_forward(x, logits, k, wgu, wd, inter="f32"):
    """Whole routed-expert layer, every stage returned.

    ``x`` float32 [T, H] (bf16 widened), ``logits`` float32 [T, E], ``wgu`` a
    quantized stack ``(q, s, g)`` for gate_up [E, 2I, H], ``wd`` for down [E, H, I].
    The intermediate h is rounded to float32 before its quantization (the
    activation fed to a quantized linear is a float32 tensor).  ``inter="bf16"``
    stores h and y in bfloat16 instead: h and y are then rounded once more, from
    float32 to bfloat16, before the quantizer and the combine read them; the
    returned ``h`` and ``y`` are the stored values.
    """
    if inter not in ("f32", "bf16"):
        raise ValueError("inter must be 'f32' or 'bf16'")
    E = np.asarray(logits).shape[1]
    ids, w = route(logits, k)
    offsets, src_row, inv = permute(ids, E)
    xq = quantize(x)
    gu = grouped_gemm(*xq, src_row, offsets, *wgu)
    h = silu_gate(gu)
    if inter == "bf16":
        h = round_to_bf16(h.astype(np.float32)).astype(np.float64)
    hq = quantize(h.astype(np.float32))
    y = grouped_gemm(*hq, None, offsets, *wd)
    if inter == "bf16":
        y = round_to_bf16(y.astype(np.float32)).astype(np.float64)
    out = combine(y, w, inv)
    return dict(topk_ids=ids, topk_w=w, offsets=offsets, src_row=src_row, inv=inv,
                xq=xq, gu=gu, h=h, hq=hq, y=y, out=out)
