"""GPU parity of the routed-expert path (route, grouped GEMM, combine) against
the oracle.

* Routing: top-k ids, expert offsets, src_row and inv bit-exact (both sides
  compare the same float32 logits); softmax weights to 1e-6 relative.
* Grouped GEMM (plain and SiLU-gated): operands are seeded random NVFP4
  tensors (random code bytes, random E4M3 scales, random global scales), so the
  oracle needs no quantization; output rows within 1e-3 relative Frobenius
  error.  At the full workload shapes the oracle checks sampled experts (the
  hottest, a cold one, and others).
* Combine: float32 routed-row outputs and weights from the seeded generator;
  bf16 output compared with the oracle rounded to bf16.
* Whole layer (reduced sizes), stage by stage, each stage given the GPU's own
  input to it: routing, X and the quantize of h bit-exact; h, y and the
  combined output within 1e-3.  The error of the output against the oracle's
  own layer end to end is printed for information: the two compute h in
  float32 vs float64, so a few codes of the quantized h may round the other way.
  Full-size stage-wise parity of both expert workloads: test_gpu_configs.py.
"""

import numpy as np
import pytest
import torch

from oracle import gemm as OG
from oracle import moe as OM
from oracle import nvfp4 as OQ
from moe_nvfp4_quantize_amd import workloads as W

import oracle_pool as OP

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def B():
    from moe_nvfp4_quantize_amd import nvfp4
    nvfp4.load_library()
    return nvfp4


def _np(t):
    return t.detach().cpu().numpy()


def _bf16_round(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.bfloat16).double().numpy()


# ---------------------------------------------------------------- routing


def _check_route(B, logits, k):
    r = B.nvfp4_moe_route(logits, k)
    torch.cuda.synchronize()
    lh = _np(logits)
    ids, w = OM.route(lh, k)
    offsets, src_row, inv = OM.permute(ids, lh.shape[1])
    np.testing.assert_array_equal(_np(r["topk_ids"]), ids)
    np.testing.assert_allclose(_np(r["topk_w"]), w, rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(_np(r["offsets"]), offsets)
    np.testing.assert_array_equal(_np(r["src_row"]), src_row)
    np.testing.assert_array_equal(_np(r["inv"]), inv)
    return r, offsets


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 3, 3), (63, 8, 2), (64, 8, 2), (65, 16, 4),
                                   (300, 1024, 32), (1000, 40, 7)])
def test_route_small(B, T, E, k):
    logits = W.random_matrix(T, E, seed=T + E + k, device="cuda")
    _check_route(B, logits, k)


# Many tokens: the counting sort's per-group counts (64 tokens a group) span
# 1,563 and 625 groups, past the scan's 32-deep load batches; k up to the
# maximum of 32 with 1024 experts.
@pytest.mark.parametrize("T,E,k", [(100000, 64, 4), (40000, 1024, 32), (65537, 7, 7)])
def test_route_many_tokens(B, T, E, k):
    logits = W.random_matrix(T, E, seed=T + E + k, device="cuda")
    _check_route(B, logits, k)


def test_route_ties_and_signed_zero(B):
    logits = torch.zeros((70, 9), device="cuda")
    logits[3] = 1.0
    logits[5, 4] = -0.0
    logits[7, [2, 6]] = 5.0
    logits[8] = torch.tensor([0.5, -1, 0.5, 2, 2, 2, -3, 0.5, 0.5])
    _check_route(B, logits, 4)


def test_route_nan_rows_stay_in_bounds(B):
    """Router rows with NaN logits (fewer than k non-NaN ones, all-NaN rows
    included): a NaN ranks as -infinity, so every token still gets k distinct
    experts in [0, E) and the permutation stays a bijection; rows without NaN
    route exactly as the oracle does."""
    T, E, k = 300, 64, 8
    logits = W.random_matrix(T, E, seed=77, device="cuda")
    logits[0] = float("nan")
    logits[5, 3:] = float("nan")
    logits[9, ::2] = float("nan")
    logits[100:164] = float("nan")
    r = B.nvfp4_moe_route(logits, k)
    torch.cuda.synchronize()
    ids, offsets = _np(r["topk_ids"]), _np(r["offsets"]).astype(np.int64)
    assert ids.min() >= 0 and ids.max() < E
    assert all(len(set(row)) == k for row in ids)
    assert list(ids[0]) == list(range(k))
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
    np.testing.assert_array_equal(np.diff(offsets), np.bincount(ids.reshape(-1), minlength=E))
    src, inv = _np(r["src_row"]), _np(r["inv"])
    assert sorted(inv.reshape(-1)) == list(range(T * k))
    np.testing.assert_array_equal(src[inv], np.repeat(np.arange(T), k).reshape(T, k))
    lh = _np(logits)
    clean = ~np.isnan(lh).any(axis=1)
    ref_ids, _ = OM.route(lh[clean], k)
    np.testing.assert_array_equal(ids[clean], ref_ids)


def test_route_empty(B):
    r = B.nvfp4_moe_route(torch.zeros((0, 8), device="cuda"), 2)
    assert torch.all(r["offsets"] == 0)


@pytest.mark.parametrize("name", ["moe_e128_top8", "moe_e512_top10"])
def test_route_full_workloads(B, name):
    cfg = W.WORKLOADS[name]
    print(f"[moe] route {name}", flush=True)
    inp = W.moe_inputs(name, device="cuda", E=cfg["E"], H=16, I=16)  # logits only matter here
    r, offsets = _check_route(B, inp["logits"], cfg["k"])
    counts = np.diff(offsets)
    print(f"[moe] {name}: rows per expert min {counts.min()} mean {counts.mean():.0f} max {counts.max()}")
    if cfg["hot"]:
        assert counts.max() > 3 * counts.mean()  # the hot-expert skew is visible


# ----------------------------------------------------------- grouped GEMM


def _rand_nvfp4(gen, shape, device, scale_lo=0x30, scale_hi=0x41):
    """Random NVFP4 tensor(s) [..., rows, K]: uniform code bytes, scales in [0.5, 2.25]."""
    *lead, rows, K = shape
    q = torch.randint(0, 256, (*lead, rows, K // 2), generator=gen, device=device, dtype=torch.uint8)
    s = torch.randint(scale_lo, scale_hi, (*lead, rows, K // 16), generator=gen, device=device,
                      dtype=torch.uint8)
    n = int(np.prod(lead)) if lead else 1
    g = (torch.rand((n,), generator=gen, device=device) + 0.5) * 2.0 ** -6
    return q, s, g


def _routing(gen, T, E, k, device, skew=False):
    logits = torch.randn((T, E), generator=gen, device=device)
    if skew:
        logits[:, :3] += 2.5
    return logits


def _grouped_case(B, T, E, k, H, N, epi, seed, sample=None, gather=True, out_dtype=torch.float32):
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    logits = _routing(gen, T, E, k, dev, skew=True)
    r = B.nvfp4_moe_route(logits, k)
    R = T * k
    a_rows = T if gather else R
    a = _rand_nvfp4(gen, (a_rows, H), dev)
    w = _rand_nvfp4(gen, (E, N, H), dev)
    out = B.nvfp4_moe_grouped_gemm(a, r["src_row"] if gather else None, r["offsets"], R, w,
                                   epilogue=epi, out_dtype=out_dtype)
    torch.cuda.synchronize()
    offsets = _np(r["offsets"]).astype(np.int64)
    src = _np(r["src_row"]) if gather else np.arange(R)
    experts = range(E) if sample is None else sample
    _check_grouped(B, a, w, out, offsets, src, experts, epi, out_dtype,
                   f"T={T} E={E} k={k} H={H} N={N} epi={epi} out={out_dtype}")
    return out, offsets


def _check_grouped(B, a, w, out, offsets, src, experts, epi, out_dtype, label):
    """Every listed expert's rows of a grouped GEMM's output against the oracle:
    relative Frobenius error at most TOL, and every element within the float32
    accumulation bound."""
    a_np = (_np(a[0]), _np(a[1]), np.float32(a[2][0].item()))
    errs, worst = [], 0.0
    for e in experts:
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        rows = src[lo:hi]
        ref = OG.gemm(a_np[0][rows], a_np[1][rows], a_np[2], _np(w[0][e]), _np(w[1][e]),
                      np.float32(w[2][e].item()))
        if epi == B.NVFP4_EPI_SILU_GATE:
            ref = OM.silu_gate(ref)
        got = _np(out[lo:hi].float()).astype(np.float64)
        if out_dtype == torch.bfloat16:
            ref = _bf16_round(ref)
        err = OG.rel_fro_error(got, ref)
        errs.append(err)
        assert err <= TOL, (e, err)
        # every element within the float32 accumulation bound (tests/oracle_pool.py)
        a_e = (a_np[0][rows], a_np[1][rows], a_np[2])
        b_e = (_np(w[0][e]), _np(w[1][e]), np.float32(w[2][e].item()))
        check = OP.silu_gate_block_check if epi == B.NVFP4_EPI_SILU_GATE else OP.gemm_block_check
        st = check(a_e, b_e, got, out_dtype == torch.bfloat16)
        worst = max(worst, st["max_ratio"])
        assert st["bad"] == 0, (e, st["bad"], st["max_ratio"])
    assert errs, "no expert had rows"
    print(f"[moe] grouped {label}: experts checked {len(errs)}, "
          f"max rel err {max(errs):.2e}, element-wise max ratio to the bound {worst:.3f}", flush=True)


# Rows per expert decide the grouped kernel's tile height (128, 192 or 256
# rows): about 60, 125, 150 and 1000 rows per expert below cover all three.
@pytest.mark.parametrize("epi", [0, 1])
@pytest.mark.parametrize("T,E,k,H,N", [(200, 7, 2, 256, 256), (37, 5, 3, 48, 96), (500, 16, 4, 512, 384),
                                       (1, 4, 1, 256, 64), (600, 4, 1, 512, 256),
                                       (2000, 2, 1, 256, 512)])
def test_grouped_gemm_small(B, T, E, k, H, N, epi):
    _grouped_case(B, T, E, k, H, N, epi, seed=T + E + N)


# K of 1024 or 2048 and an even number of 256-column N tiles: without the SiLU
# gate and with 128- and 192-row tiles each workgroup computes two N tiles of one
# M tile in a row (the second one's first K steps fetched during the first one's
# last); the gated and the 256-row cases beside them keep one N tile each.
# Every expert is checked.
@pytest.mark.parametrize("T,E,k,H,N,epi", [(500, 16, 4, 1024, 512, 1), (600, 4, 1, 1024, 512, 0),
                                           (200, 7, 2, 2048, 1024, 1), (200, 7, 2, 2048, 1024, 0),
                                           (300, 6, 2, 1024, 2048, 0), (1000, 8, 2, 1024, 512, 1)])
def test_grouped_gemm_two_tile_walk(B, T, E, k, H, N, epi):
    _grouped_case(B, T, E, k, H, N, epi, seed=T + E + N + epi)


# bf16 output (what the layer stores) with each tile height the launcher picks:
# about 256 rows per expert take 256-row tiles (2 x 2 waves), about 160 rows
# 192-row tiles and about 60 rows 128-row tiles (1 x 4 waves); gated and not,
# K with and without the two-tile walk.  Every expert checked against the
# oracle rounded to bf16.
@pytest.mark.parametrize("T,E,k,H,N,epi", [(4096, 16, 1, 512, 512, 1), (4096, 16, 1, 512, 512, 0),
                                           (2560, 16, 1, 1024, 512, 1), (2560, 16, 1, 1024, 512, 0),
                                           (960, 16, 1, 2048, 1024, 0), (960, 16, 1, 768, 512, 1),
                                           (4096, 16, 1, 768, 1024, 0)])
def test_grouped_gemm_bf16_out(B, T, E, k, H, N, epi):
    _grouped_case(B, T, E, k, H, N, epi, seed=T + H + N + epi, out_dtype=torch.bfloat16)


def test_grouped_gemm_without_gather(B):
    _grouped_case(B, 300, 6, 2, 256, 128, 0, seed=3, gather=False)


# Rows read in place (no gather), no gate, as the layer's down projection
# runs: K of 4, 5, 6, 8, 12 and 16 steps of 128, every tile height, experts left
# empty by the skewed routing (E = 64 with k = 1), bf16 and float32 output;
# every expert checked.
@pytest.mark.parametrize("T,E,k,H,N,out", [(2048, 16, 1, 512, 1024, "bf16"), (800, 8, 2, 640, 512, "f32"),
                                           (4096, 16, 1, 768, 2048, "bf16"), (2560, 16, 1, 1024, 1024, "f32"),
                                           (960, 16, 1, 1536, 512, "bf16"), (1000, 64, 1, 2048, 768, "f32"),
                                           (3000, 5, 3, 768, 256, "bf16"), (50, 3, 2, 1024, 4096, "f32")])
def test_grouped_gemm_rows_in_place(B, T, E, k, H, N, out):
    _grouped_case(B, T, E, k, H, N, 0, seed=T + E + H, gather=False,
                  out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)


# Many experts: the kernel's expert scan gives each of its 256 threads
# ceil(E / 256) experts, so E = 1000 (routed, about 2.4 rows per expert), 3000
# and 65536 (the ABI's maximum) take 4, 12 and 256 experts per thread.  The
# last two build the segment offsets directly: most experts empty, a few with
# one to several whole tiles, rows read through an arbitrary gather list.
@pytest.mark.parametrize("epi", [0, 1])
def test_grouped_gemm_many_experts_routed(B, epi):
    _grouped_case(B, 600, 1000, 4, 256, 128, epi, seed=1000 + epi)


@pytest.mark.parametrize("E,epi,out", [(3000, 0, "f32"), (3000, 1, "bf16"), (65536, 0, "bf16")])
def test_grouped_gemm_many_experts_offsets(B, E, epi, out):
    dev = "cuda"
    H, N = 256, 128
    rng = np.random.default_rng(E + epi)
    counts = np.zeros(E, dtype=np.int64)
    busy = rng.choice(E, size=min(E, 300), replace=False)
    counts[busy] = rng.integers(1, 40, size=busy.size)
    counts[busy[:6]] = [128, 256, 300, 513, 700, 1]  # whole tiles of every height, and past them
    offsets = np.concatenate([[0], np.cumsum(counts)])
    R = int(offsets[-1])
    a_rows = 900
    src = rng.integers(0, a_rows, size=R).astype(np.int32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(E + epi)
    a = _rand_nvfp4(gen, (a_rows, H), dev)
    w = _rand_nvfp4(gen, (E, N, H), dev)
    out_dtype = torch.bfloat16 if out == "bf16" else torch.float32
    got = B.nvfp4_moe_grouped_gemm(a, torch.from_numpy(src).to(dev),
                                   torch.from_numpy(offsets.astype(np.int32)).to(dev), R, w,
                                   epilogue=epi, out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check_grouped(B, a, w, got, offsets, src, [int(e) for e in np.flatnonzero(counts)], epi, out_dtype,
                   f"offsets E={E} R={R} epi={epi} out={out}")


@pytest.mark.parametrize("layout", ["last", "first", "none"])
def test_grouped_gemm_edge_segments(B, layout):
    """All rows in the last of 700 experts (the scan's last thread holds them),
    all in the first of 5, and no routed rows at all (R = 0: nothing is written,
    the call succeeds)."""
    dev = "cuda"
    H, N = 512, 256
    E = 700 if layout == "last" else 5
    counts = np.zeros(E, dtype=np.int64)
    if layout == "last":
        counts[-1] = 333
    elif layout == "first":
        counts[0] = 1000
    offsets = np.concatenate([[0], np.cumsum(counts)])
    R = int(offsets[-1])
    gen = torch.Generator(device=dev)
    gen.manual_seed(E)
    a = _rand_nvfp4(gen, (max(R, 1), H), dev)
    w = _rand_nvfp4(gen, (E, N, H), dev)
    got = B.nvfp4_moe_grouped_gemm(a, None, torch.from_numpy(offsets.astype(np.int32)).to(dev), R, w,
                                   out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert tuple(got.shape) == (R, N)
    if R:
        _check_grouped(B, a, w, got, offsets, np.arange(R), [int(np.flatnonzero(counts)[0])], 0,
                       torch.bfloat16, f"edge segments {layout} E={E} R={R}")


@pytest.mark.parametrize("H,I", [(256, 128), (2048, 768)])
def test_silu_gate_large_gate_values(B, H, I):
    """Gate values of several hundred in magnitude: below z = -88.7 the power of
    two in the kernel's SiLU overflows to inf, and h must come out as a signed
    zero (the oracle's value is below 1e-30 there), never NaN; large positive
    gates give h = gate * up.  Whole output within 1e-3 relative Frobenius error."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(H + I)
    T, E, k = 300, 6, 2
    r = B.nvfp4_moe_route(_routing(gen, T, E, k, dev, skew=True), k)
    R = T * k
    a_q, a_s, a_g = _rand_nvfp4(gen, (T, H), dev)
    a = (a_q, a_s, a_g * 4096.0)  # GEMM outputs of a few hundred
    w = _rand_nvfp4(gen, (E, 2 * I, H), dev)
    out = B.nvfp4_moe_grouped_gemm(a, r["src_row"], r["offsets"], R, w,
                                   epilogue=B.NVFP4_EPI_SILU_GATE, out_dtype=torch.float32)
    torch.cuda.synchronize()
    offsets = _np(r["offsets"]).astype(np.int64)
    src = _np(r["src_row"])
    got_all = _np(out)
    assert np.isfinite(got_all[:R]).all()
    n_neg = 0
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        rows = src[lo:hi]
        gu = OG.gemm(a_q.cpu().numpy()[rows], a_s.cpu().numpy()[rows], np.float32(a[2][0].item()),
                     _np(w[0][e]), _np(w[1][e]), np.float32(w[2][e].item()))
        with np.errstate(over="ignore"):  # float64 e^-gate overflows below gate = -709: h = -0
            ref = OM.silu_gate(gu)
        got = got_all[lo:hi].astype(np.float64)
        assert OG.rel_fro_error(got, ref) <= TOL, e
        deep = gu[:, :I] < -100.0
        n_neg += int(deep.sum())
        assert (got[deep] == 0.0).all(), e
    assert n_neg > 0, "no gate value below -100: the case does not reach the overflow"
    big = np.abs(got_all[:R]).max()
    print(f"[moe] SiLU gate H={H} I={I}: {n_neg} gates below -100 give h = 0, "
          f"max |h| {big:.3g}", flush=True)


@pytest.mark.parametrize("name,stage", [("moe_e128_top8", "gate_up"), ("moe_e128_top8", "down"),
                                        ("moe_e512_top10", "gate_up"), ("moe_e512_top10", "down")])
def test_grouped_gemm_full_shapes_sampled(B, name, stage):
    cfg = W.WORKLOADS[name]
    T, E, k, H, I = cfg["T"], cfg["E"], cfg["k"], cfg["H"], cfg["I"]
    print(f"[moe] grouped {name} {stage}", flush=True)
    sample = [0, 1, 2, E // 2, E - 1]
    if stage == "gate_up":
        _grouped_case(B, T, E, k, H, 2 * I, 1, seed=11, sample=sample)
    else:
        _grouped_case(B, T, E, k, I, H, 0, seed=12, sample=sample, gather=False)


# ------------------------------------------- fused SiLU-gate -> NVFP4 (static)


@pytest.mark.parametrize("T,E,k,H,I,g_div", [(200, 7, 2, 256, 128, 1.0), (500, 16, 4, 512, 192, 1.0),
                                             (600, 4, 1, 512, 128, 8.0), (2000, 2, 1, 256, 256, 1.0),
                                             (500, 16, 4, 1024, 256, 1.0), (300, 6, 2, 2048, 512, 1.0)])
def test_gate_up_nvfp4_epilogue(B, T, E, k, H, I, g_div):
    """The fused epilogue's h bytes equal the oracle's static quantization of the
    unfused kernel's float32 h (same accumulation, so the same h), bit for bit.
    g_div > 1 calibrates the scale below the batch's amax: saturated blocks."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(T * 7 + E)
    logits = _routing(gen, T, E, k, dev, skew=True)
    r = B.nvfp4_moe_route(logits, k)
    R = T * k
    a = _rand_nvfp4(gen, (T, H), dev)
    w = _rand_nvfp4(gen, (E, 2 * I, H), dev)
    h32 = B.nvfp4_moe_grouped_gemm(a, r["src_row"], r["offsets"], R, w,
                                   epilogue=B.NVFP4_EPI_SILU_GATE, out_dtype=torch.float32)
    torch.cuda.synchronize()
    n = int(_np(r["offsets"])[-1])
    h_np = _np(h32[:n]).astype(np.float32)
    g_h = np.float32(OQ.global_scale(h_np) / np.float32(g_div))
    hg = torch.tensor([float(g_h)], dtype=torch.float32, device=dev)
    hq, hs, _ = B.nvfp4_moe_grouped_gemm_silu_nvfp4(a, r["src_row"], r["offsets"], R, w, hg)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = OQ.quantize(h_np, g=g_h)
    np.testing.assert_array_equal(_np(hs[:n]), s_ref)
    np.testing.assert_array_equal(_np(hq[:n]), q_ref)
    print(f"[moe] fused gate_up NVFP4 T={T} E={E} I={I} g_div={g_div}: {n} rows bit-exact, "
          f"{int((s_ref == 0x7E).sum())} blocks at scale 448", flush=True)


@pytest.mark.parametrize("epi,out", [(0, "f32"), (1, "bf16"), (1, "nvfp4")])
def test_grouped_rows_past_offsets_untouched(B, epi, out):
    """R is only an upper bound on offsets[E]: the launch is sized by R, rows
    [offsets[E], R) of the output keep what they held, and the rows before them
    are what the exact-size call computes (checked against the oracle)."""
    dev = "cuda"
    T, E, k, H, I = 300, 9, 2, 512, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(31 + epi)
    r = B.nvfp4_moe_route(_routing(gen, T, E, k, dev, skew=True), k)
    n = T * k
    R = n + 77
    a = _rand_nvfp4(gen, (T, H), dev)
    N = 2 * I if epi else I
    w = _rand_nvfp4(gen, (E, N, H), dev)
    offsets = _np(r["offsets"]).astype(np.int64)
    assert offsets[-1] == n
    if out == "nvfp4":
        h32 = B.nvfp4_moe_grouped_gemm(a, r["src_row"], r["offsets"], n, w,
                                       epilogue=B.NVFP4_EPI_SILU_GATE, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check_grouped(B, a, w, h32, offsets, _np(r["src_row"]), range(E), epi, torch.float32,
                       f"rows past offsets, h in float32 (R = {n})")
        h_np = _np(h32).astype(np.float32)
        g_h = np.float32(OQ.global_scale(h_np))
        hq = torch.full((R, I // 2), 0xAB, dtype=torch.uint8, device=dev)
        hs = torch.full((R, I // 16), 0xCD, dtype=torch.uint8, device=dev)
        B.nvfp4_moe_grouped_gemm_silu_nvfp4(a, r["src_row"], r["offsets"], R, w,
                                            torch.tensor([float(g_h)], device=dev), out=(hq, hs))
        torch.cuda.synchronize()
        q_ref, s_ref, _ = OQ.quantize(h_np, g=g_h)
        np.testing.assert_array_equal(_np(hq[:n]), q_ref)
        np.testing.assert_array_equal(_np(hs[:n]), s_ref)
        assert bool((hq[n:] == 0xAB).all()) and bool((hs[n:] == 0xCD).all())
        return
    out_dtype = torch.bfloat16 if out == "bf16" else torch.float32
    c = torch.full((R, I), float("nan"), dtype=out_dtype, device=dev)
    B.nvfp4_moe_grouped_gemm(a, r["src_row"], r["offsets"], R, w, epilogue=epi, out_dtype=out_dtype, out=c)
    torch.cuda.synchronize()
    assert bool(torch.isnan(c[n:]).all())
    assert not bool(torch.isnan(c[:n]).any())
    _check_grouped(B, a, w, c, offsets, _np(r["src_row"]), range(E), epi, out_dtype,
                   f"rows past offsets epi={epi} out={out} (R = {R}, offsets[E] = {n})")


@pytest.mark.parametrize("epi,out", [(0, "f32"), (0, "bf16"), (1, "bf16"), (1, "f32")])
def test_grouped_output_independent_of_tile_height(B, epi, out):
    """R, the host's upper bound on offsets[E], sizes the launch, and the
    launcher picks the tile height from R / E: the same 1000 routed rows over 16
    experts computed with R = 1000, 2400 and 3200 run 128-, 192- and 256-row
    tiles (the first two, without the gate, with the two-tile walk), and the
    rows come out bit-identical, each output's sum over K taken in the same
    order at every height.  The first run is checked against the oracle."""
    dev = "cuda"
    T, E, k, H = 1000, 16, 1, 1024
    N = 1024 if epi else 512
    gen = torch.Generator(device=dev)
    gen.manual_seed(57 + epi)
    r = B.nvfp4_moe_route(_routing(gen, T, E, k, dev, skew=True), k)
    a = _rand_nvfp4(gen, (T, H), dev)
    w = _rand_nvfp4(gen, (E, N, H), dev)
    out_dtype = torch.bfloat16 if out == "bf16" else torch.float32
    n = T * k
    outs = [B.nvfp4_moe_grouped_gemm(a, r["src_row"], r["offsets"], R, w, epilogue=epi,
                                     out_dtype=out_dtype)[:n] for R in (n, 150 * E, 200 * E)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    _check_grouped(B, a, w, outs[0], _np(r["offsets"]).astype(np.int64), _np(r["src_row"]), range(E),
                   epi, out_dtype, f"tile heights 128 / 192 / 256, epi={epi} out={out}")


def test_gate_up_nvfp4_epilogue_unsupported_layout(B):
    # K % 256 != 0: the fused path reports "unsupported" instead of running
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    r = B.nvfp4_moe_route(_routing(gen, 40, 4, 2, dev), 2)
    a = _rand_nvfp4(gen, (40, 48), dev)
    w = _rand_nvfp4(gen, (4, 64, 48), dev)
    hg = torch.ones(1, dtype=torch.float32, device=dev)
    with pytest.raises(B.NVFP4Error) as ei:
        B.nvfp4_moe_grouped_gemm_silu_nvfp4(a, r["src_row"], r["offsets"], 80, w, hg)
    assert ei.value.status == B.NVFP4_ERR_UNSUPPORTED


# ---------------------------------------------------------------- combine


# H % 8 != 0 (100, 1029) takes the one-element-per-thread path, the others the
# 8-wide vector path; k up to 32
@pytest.mark.parametrize("T,k,H", [(1, 1, 16), (100, 8, 2048), (33, 10, 4096 + 64), (7, 32, 100),
                                   (1000, 3, 1029)])
@pytest.mark.parametrize("y_bf16", [False, True])
def test_combine(B, T, k, H, y_bf16):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(T * k + H)
    R = T * k
    y = torch.randn((R, H), generator=gen, device="cuda")
    if y_bf16:
        y = y.to(torch.bfloat16)
    w = torch.rand((T, k), generator=gen, device="cuda")
    inv = torch.randperm(R, generator=gen, device="cuda").to(torch.int32).reshape(T, k)
    out = B.nvfp4_moe_combine(y, w, inv)
    torch.cuda.synchronize()
    ref = OM.combine(_np(y.float()), _np(w), _np(inv))
    err = OG.rel_fro_error(_np(out.float()), _bf16_round(ref))
    assert err <= TOL, err
    out32 = B.nvfp4_moe_combine(y, w, inv, out_dtype=torch.float32)
    np.testing.assert_allclose(_np(out32), ref, rtol=1e-5, atol=1e-5)
    # float32 output: exactly the arithmetic the entry point states, slot by
    # slot, each product and each addition rounded once to float32
    yf, wf, iv = _np(y.float()), _np(w), _np(inv)
    acc = np.zeros((T, H), dtype=np.float32)
    for j in range(k):
        acc = acc + wf[:, j:j + 1] * yf[iv[:, j]]
    np.testing.assert_array_equal(_np(out32), acc)


def test_combine_bf16_output_is_rounded_f32_output(B):
    """bf16 output = the float32 combine rounded to nearest even, bit for bit,
    subnormal sums included."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    T, k, H = 64, 8, 4096
    y = torch.randn((T * k, H), generator=gen, device="cuda")
    y[: T * k // 2] *= 2.0 ** -130  # subnormal products
    w = torch.rand((T, k), generator=gen, device="cuda")
    inv = torch.randperm(T * k, generator=gen, device="cuda").to(torch.int32).reshape(T, k)
    o32 = B.nvfp4_moe_combine(y, w, inv, out_dtype=torch.float32)
    o16 = B.nvfp4_moe_combine(y, w, inv, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16.cpu().view(torch.int16), o32.cpu().to(torch.bfloat16).view(torch.int16))


# ------------------------------------------------------------- end to end


@pytest.mark.parametrize("T,E,k,H,I,hot", [(256, 16, 4, 512, 256, 0), (512, 64, 8, 256, 128, 4),
                                           (96, 8, 1, 256, 64, 0)])
@pytest.mark.parametrize("inter", ["f32", "bf16"])
def test_layer_end_to_end(B, T, E, k, H, I, hot, inter):
    inp = W.moe_inputs("moe_e512_top10", device="cuda", T=T, E=E, k=k, H=H, I=I, hot=hot)
    wgu = B.nvfp4_quantize_batched(inp["w_gate_up"])
    wd = B.nvfp4_quantize_batched(inp["w_down"])
    res = B.moe_layer(inp["x"], inp["logits"], k, wgu, wd, keep=True,
                      inter_dtype=torch.bfloat16 if inter == "bf16" else torch.float32)
    torch.cuda.synchronize()
    qgu = OM.quantize_experts(_np(inp["w_gate_up"].float()))
    qd = OM.quantize_experts(_np(inp["w_down"].float()))
    # the GPU's offline weight quantization is bit-exact
    for got, ref in zip(wgu + wd, qgu + qd):
        np.testing.assert_array_equal(_np(got), ref)
    ref = OM.moe_forward(_np(inp["x"].float()), _np(inp["logits"]), k, qgu, qd, inter=inter)
    np.testing.assert_array_equal(_np(res["topk_ids"]), ref["topk_ids"])
    np.testing.assert_array_equal(_np(res["src_row"]), ref["src_row"])
    for got, want in zip(res["xq"], ref["xq"]):
        np.testing.assert_array_equal(_np(got).reshape(np.shape(want)), want)
    # stage by stage, each given the GPU's own input to it
    rnd = _bf16_round if inter == "bf16" else (lambda v: v)
    h_err = OG.rel_fro_error(_np(res["h"].float()).astype(np.float64), ref["h"])  # same quantized inputs
    h_gpu = _np(res["h"].float())
    hq_ref = OQ.quantize(h_gpu)
    for got, want in zip(res["hq"], hq_ref):
        np.testing.assert_array_equal(_np(got).reshape(np.shape(want)), want)
    y_ref = rnd(OM.grouped_gemm(*hq_ref, None, ref["offsets"], *qd))
    y_err = OG.rel_fro_error(_np(res["y"].float()).astype(np.float64), y_ref)
    out_ref = OM.combine(_np(res["y"].float()), _np(res["topk_w"]), _np(res["inv"]))
    out_err = OG.rel_fro_error(_np(res["out"].float()), _bf16_round(out_ref))
    # end to end against the oracle's own layer (information: its float64 h may
    # round a code of the quantized h the other way)
    e2e = OG.rel_fro_error(_np(res["out"].float()), _bf16_round(ref["out"]))
    same = np.mean(OQ.unpack_codes(_np(res["hq"][0])) == OQ.unpack_codes(ref["hq"][0]))
    print(f"[moe] layer T={T} E={E} k={k} {inter}: h {h_err:.2e}, hq bit-exact, y {y_err:.2e}, "
          f"out {out_err:.2e}; end to end {e2e:.2e} (hq codes equal to the oracle's own {same:.5f})",
          flush=True)
    assert h_err <= TOL and y_err <= TOL and out_err <= TOL
