"""Pins for oracle.gemm and oracle.moe.  No GPU.

GEMM: exact rational brute force on tiny non-square operands (catches a
transposed operand or a dropped scale), a closed form on crafted operands, and
linearity in the global scales.

MoE: top-k by brute force over all subsets, closed-form softmax weights,
permutation invariants, SiLU closed forms, and two reductions -- one expert with
k = 1 is the dense NVFP4 MLP, and identical experts make the output independent
of the routing.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm as G
from oracle import moe as M
from oracle import nvfp4 as Q
from oracle.formats import e2m1_decode, e4m3_decode


def _rand_q(rng, rows, cols):
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.standard_normal((rows, 1)))).astype(np.float32)
    return Q.quantize(x)


def test_gemm_equals_exact_brute_force():
    rng = np.random.default_rng(0)
    Mr, N, K = 3, 5, 48
    a = _rand_q(rng, Mr, K)
    b = _rand_q(rng, N, K)
    y = G.gemm(*a, *b)
    assert y.shape == (Mr, N)
    ca, cb = Q.unpack_codes(a[0]), Q.unpack_codes(b[0])
    for i in range(Mr):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                va = Fraction(float(e2m1_decode(ca[i, k]))) * Fraction(float(e4m3_decode(a[1][i, k // 16])))
                vb = Fraction(float(e2m1_decode(cb[j, k]))) * Fraction(float(e4m3_decode(b[1][j, k // 16])))
                acc += va * vb
            acc *= Fraction(float(a[2])) * Fraction(float(b[2]))
            assert abs(Fraction(float(y[i, j])) - acc) <= abs(acc) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 200)


def test_gemm_closed_form_all_ones():
    """Codes 2 (= 1.0), scales 1.0 (0x38), g = 1: every output is K."""
    K = 64
    a = (np.full((4, K // 2), 0x22, np.uint8), np.full((4, K // 16), 0x38, np.uint8), np.float32(1))
    b = (np.full((6, K // 2), 0x22, np.uint8), np.full((6, K // 16), 0x38, np.uint8), np.float32(2))
    np.testing.assert_array_equal(G.gemm(*a, *b), np.full((4, 6), 2.0 * K))


def test_gemm_scales_enter_linearly():
    rng = np.random.default_rng(1)
    a = _rand_q(rng, 4, 32)
    b = _rand_q(rng, 7, 32)
    y = G.gemm(*a, *b)
    y2 = G.gemm(a[0], a[1], np.float32(a[2] * 2), b[0], b[1], np.float32(b[2] * 8))
    np.testing.assert_array_equal(y2, y * 16)
    sub = G.gemm_rows(*a, *b, rows=[1, 3], cols=[0, 6])
    np.testing.assert_allclose(sub, y[np.ix_([1, 3], [0, 6])], rtol=1e-14)


def test_rel_fro_error():
    assert G.rel_fro_error([[3.0, 4.0]], [[3.0, 4.0]]) == 0.0
    assert math.isclose(G.rel_fro_error([[3.0, 4.5]], [[3.0, 4.0]]), 0.1)


# ------------------------------------------------------------------ MoE


def test_topk_brute_force():
    rng = np.random.default_rng(2)
    T, E, k = 20, 7, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :] = 0.5  # all equal: lowest ids win, in id order
    logits[1, [2, 5]] = 9.0  # a tie at the top
    ids, sel = M.topk(logits, k)
    for t in range(T):
        best = None
        for subset in itertools.combinations(range(E), k):
            key = sorted(subset, key=lambda e: (-logits[t, e], e))
            score = [(-logits[t, e], e) for e in key]
            if best is None or score < best[0]:
                best = (score, key)
        assert list(ids[t]) == best[1]
    assert list(ids[0]) == [0, 1, 2] and list(ids[1][:2]) == [2, 5]


def test_softmax_weights_closed_forms():
    sel = np.array([[1.5, -0.25], [3.0, 3.0]], dtype=np.float32)
    w = M.softmax_weights(sel)
    assert math.isclose(w[0, 0], 1 / (1 + math.exp(-1.75)), rel_tol=1e-15)
    assert w[1, 0] == w[1, 1] == 0.5
    rng = np.random.default_rng(3)
    w = M.softmax_weights(rng.standard_normal((50, 10)).astype(np.float32))
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-15)
    assert np.all(M.softmax_weights(np.zeros((3, 1), np.float32)) == 1.0)


def test_route_equals_full_softmax_renormalised():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((30, 16)).astype(np.float32)
    ids, w = M.route(logits, 4)
    full = np.exp(logits.astype(np.float64))
    full /= full.sum(1, keepdims=True)
    pick = np.take_along_axis(full, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, pick / pick.sum(1, keepdims=True), rtol=1e-13)


def test_permute_invariants():
    rng = np.random.default_rng(5)
    T, E, k = 40, 9, 3
    ids, _ = M.route(rng.standard_normal((T, E)).astype(np.float32), k)
    offsets, src_row, inv = M.permute(ids, E)
    R = T * k
    assert offsets[0] == 0 and offsets[-1] == R and np.all(np.diff(offsets) >= 0)
    np.testing.assert_array_equal(np.diff(offsets), np.bincount(ids.reshape(-1), minlength=E))
    assert sorted(inv.reshape(-1)) == list(range(R))  # a bijection
    for t in range(T):
        for j in range(k):
            r = inv[t, j]
            e = ids[t, j]
            assert offsets[e] <= r < offsets[e + 1] and src_row[r] == t
    for e in range(E):  # ascending tokens inside an expert
        seg = src_row[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_silu_gate_closed_forms():
    gu = np.array([[0.0, 1.0, 7.0, 2.0], [50.0, -50.0, 1.0, 1.0]])
    h = M.silu_gate(gu)
    assert h.shape == (2, 2)
    assert h[0, 0] == 0.0
    assert math.isclose(h[0, 1], 1.0 / (1.0 + math.exp(-1.0)) * 2.0, rel_tol=1e-15)
    assert math.isclose(h[1, 0], 50.0, rel_tol=1e-15)
    assert abs(h[1, 1]) < 1e-20


def test_combine_picks_weighted_rows():
    y = np.arange(12, dtype=np.float64).reshape(4, 3)
    inv = np.array([[2, 0], [1, 3]])
    w = np.array([[1.0, 0.0], [0.25, 0.75]])
    out = M.combine(y, w, inv)
    np.testing.assert_array_equal(out[0], y[2])
    np.testing.assert_array_equal(out[1], 0.25 * y[1] + 0.75 * y[3])


def _experts(rng, E, I, H, same=False):
    wgu = (rng.standard_normal((1 if same else E, 2 * I, H)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((1 if same else E, H, I)) * 0.05).astype(np.float32)
    if same:
        wgu = np.repeat(wgu, E, 0)
        wd = np.repeat(wd, E, 0)
    return wgu, wd


def _dense_mlp(x, wgu, wd):
    """The dense NVFP4 MLP written directly from the pieces (no grouping)."""
    xq = Q.quantize(x)
    gq = Q.quantize(wgu)
    dq = Q.quantize(wd)
    gu = Q.dequantize(*xq) @ Q.dequantize(*gq).T
    i = wgu.shape[0] // 2
    h = gu[:, :i] / (1 + np.exp(-gu[:, :i])) * gu[:, i:]
    hq = Q.quantize(h.astype(np.float32))
    return Q.dequantize(*hq) @ Q.dequantize(*dq).T


def test_single_expert_is_dense_mlp():
    rng = np.random.default_rng(6)
    T, H, I = 12, 32, 16
    x = rng.standard_normal((T, H)).astype(np.float32)
    wgu, wd = _experts(rng, 1, I, H)
    res = M.moe_forward(x, rng.standard_normal((T, 1)).astype(np.float32), 1,
                        M.quantize_experts(wgu), M.quantize_experts(wd))
    np.testing.assert_array_equal(res["topk_w"], 1.0)
    np.testing.assert_allclose(res["out"], _dense_mlp(x, wgu[0], wd[0]), rtol=1e-12, atol=1e-14)


def test_identical_experts_ignore_routing():
    rng = np.random.default_rng(7)
    T, H, I, E, k = 16, 32, 16, 5, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wgu, wd = _experts(rng, E, I, H, same=True)
    qgu, qd = M.quantize_experts(wgu), M.quantize_experts(wd)
    out1 = M.moe_forward(x, rng.standard_normal((T, E)).astype(np.float32), k, qgu, qd)["out"]
    out2 = M.moe_forward(x, rng.standard_normal((T, E)).astype(np.float32), k, qgu, qd)["out"]
    np.testing.assert_allclose(out1, out2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out1, _dense_mlp(x, wgu[0], wd[0]), rtol=1e-12, atol=1e-14)


def test_grouped_gemm_empty_experts_and_gather():
    rng = np.random.default_rng(8)
    a = _rand_q(rng, 6, 32)
    w = M.quantize_experts((rng.standard_normal((3, 4, 32))).astype(np.float32))
    offsets = np.array([0, 0, 5, 5])  # experts 0 and 2 empty
    src = np.array([5, 0, 3, 3, 1])
    y = M.grouped_gemm(*a, src, offsets, *w)
    ref = Q.dequantize(*a)[src] @ Q.dequantize(w[0][1], w[1][1], w[2][1]).T
    np.testing.assert_allclose(y, ref, rtol=1e-14)


def test_bf16_intermediates_round_through_torch_bfloat16():
    """With inter="bf16" the stored h and y are torch's bfloat16 casts of the
    float32 values of the float32 path's stages, and the output is their combine."""
    import torch
    rng = np.random.default_rng(9)
    T, H, I, E, k = 24, 64, 32, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wgu, wd = _experts(rng, E, I, H)
    qgu, qd = M.quantize_experts(wgu), M.quantize_experts(wd)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ref = M.moe_forward(x, logits, k, qgu, qd)
    got = M.moe_forward(x, logits, k, qgu, qd, inter="bf16")

    def bf(v):
        return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got["h"], bf(ref["h"]))
    hq = Q.quantize(bf(ref["h"]).astype(np.float32))
    for a, b in zip(got["hq"], hq):
        np.testing.assert_array_equal(a, b)
    y = M.grouped_gemm(*hq, None, ref["offsets"], *qd)
    np.testing.assert_array_equal(got["y"], bf(y))
    np.testing.assert_array_equal(got["out"], M.combine(bf(y), ref["topk_w"], ref["inv"]))
    with pytest.raises(ValueError):
        M.moe_forward(x, logits, k, qgu, qd, inter="f16")
