"""Pins of the quantizer's float32 operation order against exact division.  No GPU.

The pages fix the format (two-level scaling page, section "Core: the W4A4
two-level scaling mechanism": E2M1 codes of x scaled by its block's E4M3 scale
and the tensor's FP32 global scale) but no order of float32 operations.  The
oracle takes one reading (one rounding at a time, all float32):

  block scale   s = E4M3(fl(bmax / fl(6 g)))            (steps 3-4)
  element code  code = E2M1(fl(x * fl(1 / fl(s g))))    (steps 5-6)

Against these stands the plain definition: the E4M3 code nearest the exact
quotient bmax / (6 g), and the E2M1 code nearest the exact quotient x / (s g),
both round to nearest even, saturating.  Here the exact codes are computed
without any division: a code is fixed by where |x| lies among the midpoints of
the grid times the divisor, and every such product is exact in float64 (an
E2M1 midpoint has at most 3 significant bits, an E4M3 scale 4, an E4M3
midpoint 5, 6 has 2 and g 24: at most 31 bits), as are the float32 inputs.
Exact rational arithmetic confirms that claim on a sample.

The two readings may only disagree where the exact quotient lies within the
float32 rounding of the oracle's steps of a midpoint: three roundings move the
element quotient by at most (1 + 2^-24)^3 - 1 < 4 * 2^-24 relative, two move the
scale quotient by at most 3 * 2^-24.  The tests assert exactly that, on the
linear workload in full and on rows of every other workload's tensors, and
report how many codes each reading decides (the counts are recorded in the
design notes).  Likewise for the four-over-six choice: the float32 error sums
may only pick a different candidate than exact (rational) error sums where the
two sums lie within float32 summation error of each other.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import four_over_six as F46
from oracle import nvfp4 as Q
from oracle.formats import E4M3_NONNEG, e2m1_decode, e4m3_decode
from moe_nvfp4_quantize_amd import workloads as W

U = 2.0 ** -24
E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
E4M3_MIDS = (E4M3_NONNEG[1:] + E4M3_NONNEG[:-1]) / 2  # 126 midpoints, the last 416


def _round_by_midpoints(a, mids, unit):
    """Index (ties to even) of the nearest grid point to a / unit, from exact
    comparisons of a against mids * unit (all float64-exact).  a >= 0."""
    prod = mids[None, :] * unit[:, None]
    above = (a[:, None] > prod).sum(axis=1)
    tie = (a[:, None] == prod).any(axis=1)
    # at a tie the two neighbours are `above` and `above + 1`: take the even one
    return np.where(tie & (above % 2 == 1), above + 1, above)


def exact_element_codes(x, s, g):
    """E2M1 magnitude code (0..7) of x / (e4m3(s) g), exact, saturating at 6."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    sg = (e4m3_decode(s).astype(np.float64) * np.float64(g))          # exact
    unit = np.repeat(sg, 16, axis=1).reshape(-1)
    return _round_by_midpoints(np.abs(x.astype(np.float64)).reshape(-1), E2M1_MIDS, unit).reshape(rows, cols)


def exact_block_scales(x, g):
    """E4M3 code of min(bmax / (6 g), 448), exact, a zero raised to code 1."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    bmax = np.abs(x.astype(np.float64)).reshape(rows, cols // 16, 16).max(axis=-1).reshape(-1)
    six_g = np.full(bmax.shape, 6.0 * np.float64(g))                   # exact
    code = _round_by_midpoints(bmax, E4M3_MIDS, six_g)                 # 126 = 448 also for > 448
    return np.maximum(code, 1).reshape(rows, cols // 16)


def _nearest_mid_gap(a, mids, unit):
    """min over midpoints m of |a - m * unit| / a (float64)."""
    prod = mids[None, :] * unit[:, None]
    return np.abs(a[:, None] - prod).min(axis=1) / np.maximum(a, np.finfo(np.float64).tiny)


def test_midpoint_products_are_exact_in_float64():
    """The float64 products the exact codes rest on equal the rational ones."""
    rng = np.random.default_rng(0)
    gs = (np.exp(rng.uniform(np.log(1e-9), np.log(10.0), 400)) / 2688).astype(np.float32)
    for g in gs[:200]:
        for sc in rng.integers(1, 127, 4):
            sv = float(e4m3_decode(sc))
            for m in E2M1_MIDS:
                assert Fraction(m * sv * float(g)) == Fraction(m) * Fraction(sv) * Fraction(float(g))
    for g in gs[200:]:
        for m in rng.choice(E4M3_MIDS, 8):
            assert Fraction(m * (6.0 * float(g))) == Fraction(float(m)) * 6 * Fraction(float(g))


def test_exact_codes_against_rational_division():
    """exact_element_codes / exact_block_scales equal a nearest search in
    rationals (Fractions) on values placed at, and next to, midpoints."""
    rng = np.random.default_rng(1)
    g = np.float32(0.0123)
    s = rng.integers(0x20, 0x60, (4, 2)).astype(np.uint8)
    unit = np.repeat(e4m3_decode(s) * float(g), 16, axis=1)
    base = rng.choice(np.concatenate([E2M1_MIDS, [0.5, 1, 3, 6, 7.5]]), (4, 32)) * unit
    x = base.astype(np.float32)
    x[:, ::3] = np.nextafter(x[:, ::3], np.float32(np.inf))
    x[:, 1::3] = np.nextafter(x[:, 1::3], np.float32(0))
    x[:, 5] = -x[:, 5]
    grid = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    got = exact_element_codes(x, s, g)
    for r in range(4):
        for c in range(32):
            y = min(abs(Fraction(float(x[r, c]))) / (Fraction(float(e4m3_decode(s[r, c // 16]))) * Fraction(float(g))),
                    Fraction(6))
            d = [abs(y - v) for v in grid]
            best = [i for i in range(8) if d[i] == min(d)]
            want = best[0] if len(best) == 1 else [i for i in best if i % 2 == 0][0]
            assert got[r, c] == want, (r, c, float(y))
    # block scales: block maxima at and next to E4M3 midpoints times 6g
    mids = rng.choice(E4M3_MIDS, 64)
    bm = (mids * 6.0 * float(g)).astype(np.float32)
    bm[::2] = np.nextafter(bm[::2], np.float32(np.inf))
    xs = np.zeros((1, 16 * 64), np.float32)
    xs[0, ::16] = bm
    got_s = exact_block_scales(xs, g)[0]
    table = [Fraction(float(v)) for v in E4M3_NONNEG]
    for b in range(64):
        t = min(Fraction(float(bm[b])) / (6 * Fraction(float(g))), Fraction(448))
        d = [abs(t - v) for v in table]
        best = [i for i in range(len(table)) if d[i] == min(d)]
        want = best[0] if len(best) == 1 else [i for i in best if i % 2 == 0][0]
        assert got_s[b] == max(want, 1), b


def test_planted_division_order_is_caught():
    """The op order is a real choice: on values built at E2M1 midpoints times
    a global scale whose products with the block scale are not float32 values,
    the oracle's reciprocal-multiply reading and exact division decide some
    codes differently, each one within float32 rounding of its midpoint."""
    g = np.float32(1.0 / 3.0)  # s g not representable: every rounding step matters
    s = np.full((1, 64), 0x38, np.uint8)  # scale 1.0
    x = np.zeros((1, 1024), np.float32)
    # one block max = 6 s g keeps the block scale at 1.0 (bmax / 6g = 1 exactly in reals)
    x[0, ::16] = np.float32(6.0 * float(np.float32(g)))
    mids = np.tile(E2M1_MIDS, 150)[:960]
    body = (mids * float(g)).astype(np.float32)
    mask = np.ones(1024, bool)
    mask[::16] = False
    x[0, mask] = body
    q, s_o, g_o = Q.quantize(x, g=g)
    codes = Q.unpack_codes(q)[0] & 7
    exact = exact_element_codes(x, s_o, g_o)[0]
    n_diff = int((codes != exact).sum())
    assert n_diff > 0
    a = np.abs(x[0].astype(np.float64))
    sg = np.repeat(e4m3_decode(s_o[0]) * np.float64(g_o), 16)
    gap = _nearest_mid_gap(a[codes != exact], E2M1_MIDS, sg[codes != exact])
    assert np.all(gap <= 4 * U)


def compare_with_g(x, g):
    """(elements, differing codes, blocks, differing scales) for rows x of a
    tensor whose global scale is g; asserts every disagreement between the
    oracle's float32 order and exact division lies within float32 rounding of
    a midpoint and moves the code by one step.  Row chunks bound the memory."""
    n = dc_tot = nb = ds_tot = 0
    for r0 in range(0, x.shape[0], 256):
        xc = x[r0:r0 + 256]
        rows, cols = xc.shape
        q, s, _ = Q.quantize(xc, g=g)
        s_exact = exact_block_scales(xc, g)
        ds = s != s_exact
        if ds.any():
            bmax = np.abs(xc.astype(np.float64)).reshape(rows, cols // 16, 16).max(axis=-1)[ds]
            gap = _nearest_mid_gap(bmax, E4M3_MIDS, np.full(bmax.shape, 6.0 * np.float64(g)))
            assert np.all(gap <= 3 * U), gap.max()
            assert np.all(np.abs(s[ds].astype(int) - s_exact[ds].astype(int)) == 1)
        codes = Q.unpack_codes(q)
        assert np.array_equal(codes >> 3, np.signbit(xc).astype(np.uint8))
        mag = (codes & 7).astype(np.int64)
        mag_exact = exact_element_codes(xc, s, g)
        dc = mag != mag_exact
        if dc.any():
            a = np.abs(xc.astype(np.float64))[dc]
            sg = np.repeat(e4m3_decode(s).astype(np.float64) * np.float64(g), 16, axis=1)[dc]
            assert np.all(_nearest_mid_gap(a, E2M1_MIDS, sg) <= 4 * U)
            assert np.all(np.abs(mag[dc] - mag_exact[dc]) == 1)
        n += xc.size
        dc_tot += int(dc.sum())
        nb += s.size
        ds_tot += int(ds.sum())
    return n, dc_tot, nb, ds_tot


def _workload_tensors():
    """(label, float32 rows, global scale of the whole tensor) of every
    workload, drawn on the CPU with the workload's distributions: activations
    in full except the two largest (2048 rows each), 512 rows of each weight."""
    out = []
    x, w = W.linear_inputs("linear_16x512")
    out += [("linear_16x512 X (all)", x.numpy()), ("linear_16x512 W (all)", w.numpy())]
    x, w = W.linear_inputs("prefill_8192x5120")
    xf, wf = x.float().numpy(), w.float().numpy()
    out += [("prefill_8192x5120 X (2048 of 8192 rows)", xf, np.r_[0:1024, 7168:8192]),
            ("prefill_8192x5120 W (512 of 25600 rows)", wf, np.r_[0:256, 25344:25600])]
    x, w = W.linear_inputs("lmhead_128x151936")
    out += [("lmhead_128x151936 X (all)", x.float().numpy()),
            ("lmhead_128x151936 W (512 of 151936 rows)", w.float().numpy(), np.r_[0:256, 151680:151936])]
    d = W.moe_inputs("moe_e128_top8", weights=False)
    out.append(("moe_e128_top8 X (all)", d["x"].float().numpy()))
    d = W.moe_inputs("moe_e512_top10", weights=False)
    out.append(("moe_e512_top10 X (2048 of 8192 rows)", d["x"].float().numpy(), np.r_[0:1024, 7168:8192]))
    return out


@pytest.fixture(scope="module")
def workload_counts():
    res = {}
    for item in _workload_tensors():
        label, t = item[0], item[1]
        g = Q.global_scale(t)
        rows = t if len(item) == 2 else t[item[2]]
        res[label] = compare_with_g(rows, g)
    print()
    print("| tensor | elements | codes the op order decides | blocks | scales the op order decides |")
    for label, (n, dc, nb, ds) in res.items():
        print(f"| {label} | {n:,} | {dc:,} ({dc / n:.2e}) | {nb:,} | {ds:,} ({ds / nb:.2e}) |")
    return res


def test_workloads_disagree_only_near_midpoints(workload_counts):
    """Every workload tensor: all disagreements bounded (asserted inside
    compare_with_g); the counts are the table in the design notes."""
    assert sum(v[0] for v in workload_counts.values()) > 2 * 10 ** 7


# ------------------------------------------------------------ four-over-six


def _exact_block_error(x_blk, codes_blk, sc, g):
    """Sum over the block of (x - e2m1 * e4m3 * g)^2 in rationals."""
    G = Fraction(float(g))
    sv = Fraction(float(e4m3_decode(sc)))
    tot = Fraction(0)
    for xv, c in zip(x_blk, codes_blk):
        d = Fraction(float(xv)) - Fraction(float(e2m1_decode(c))) * sv * G
        tot += d * d
    return tot


def test_four_over_six_choice_against_exact_errors():
    """The float32 error sums pick the same candidate as exact ones except
    where the exact sums lie within float32 summation error of each other;
    counts of both reported."""
    rows = []
    x, w = W.linear_inputs("linear_16x512")
    rows.append(("linear_16x512 W", w.numpy()))
    _, w = W.linear_inputs("prefill_8192x5120")
    wf = w.float().numpy()
    g_pref = Q.global_scale(wf)
    rows.append(("prefill W rows", wf[np.r_[0:16, 25584:25600]]))
    del w, wf
    print()
    decided = 0
    for label, t in rows:
        g = Q.global_scale(t) if label.startswith("linear") else g_pref
        q, s, _, took4 = F46.quantize(t, g=g)
        r, c = t.shape
        s6, s4 = F46.candidate_scales(t, g, 6), F46.candidate_scales(t, g, 4)
        c6, c4 = Q.encode_elements(t, s6, g), Q.encode_elements(t, s4, g)
        e6 = F46.block_errors(t, c6, s6, g).astype(np.float64)
        e4 = F46.block_errors(t, c4, s4, g).astype(np.float64)
        # float64 errors first; blocks whose float32 sums sit close get exact sums
        close = np.abs(e4 - e6) <= 64 * U * np.maximum(e4, e6)
        n_close = 0
        for i, j in zip(*np.nonzero(close)):
            n_close += 1
            xb = t[i, 16 * j:16 * j + 16]
            ex6 = _exact_block_error(xb, c6[i, 16 * j:16 * j + 16], s6[i, j], g)
            ex4 = _exact_block_error(xb, c4[i, 16 * j:16 * j + 16], s4[i, j], g)
            exact4 = ex4 < ex6
            if exact4 != took4[i, j]:
                decided += 1
                # float32 accumulation of 16 squares: error well within 24 units
                assert abs(float(ex4 - ex6)) <= 24 * U * float(max(ex4, ex6))
        far = ~close
        # away from near-ties the float64 sums (within 1e-15 of the exact ones) decide
        xd6 = np.zeros_like(e6)
        xd4 = np.zeros_like(e4)
        for (cc, ss, out) in ((c6, s6, xd6), (c4, s4, xd4)):
            v = (e2m1_decode(cc).reshape(r, c // 16, 16) * e4m3_decode(ss)[..., None]) * np.float64(g)
            d = t.reshape(r, c // 16, 16).astype(np.float64) - v
            out[...] = (d * d).sum(axis=-1)
        assert np.array_equal((xd4 < xd6)[far], took4[far]), label
        print(f"[4/6] {label}: {t.size // 16} blocks, {int(took4.sum())} take 4, {n_close} near-ties "
              f"checked exactly, {decided} decided by float32 rounding")
