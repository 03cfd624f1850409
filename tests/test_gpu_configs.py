"""Parity at the full sizes of the four large workloads, every element.

* Quantize: codes, scales and global scale of the whole tensor bit-exact
  against the oracle (prefill X and W, lm_head X and W, both MoE X), the oracle
  run over row blocks in a process pool (tests/oracle_pool.py).
* Dense GEMM (prefill 8192x5120x25600, lm_head 128x151936x2048, bf16 out): the
  whole output against the oracle's float64 product of its own quantized
  operands; relative Frobenius error <= 1e-3 against the oracle rounded to
  bf16, and every element within the float32 accumulation bound plus one bf16
  unit (oracle_pool's module docstring states the bound).
* Dynamic quantize at the single-read path's capacity and one row past it
  (the two-pass path), bf16 and float32, every code and scale bit-exact.
* Static-scale quantize of the prefill X (a calibrated scale, and one that
  saturates), every code and scale bit-exact.
* Quantize-dequantize of the prefill X and W (single-read and two-pass
  paths), every value bit-exact.
* Four-over-six offline quantize of the prefill and lm_head weights, every
  code and scale bit-exact.
* FP8 W8A8 on the prefill workload: E4M3 codes and per-tensor scales of X and
  W bit-exact, the whole bf16 GEMM output within its float32 summation bound.
* MoE (128 experts top-8, 512 experts top-10), stage by stage, each stage given
  the GPU's own input to it (the float32/bf16 h and y are computed in a
  different precision than the oracle's float64 ones, so a downstream code may
  round the other way; every stage is exact or within its own bound):
  routing bit-exact; X quantize bit-exact; offline expert weights bit-exact
  (every expert of the 128, sampled experts of the 512: the 16 hottest and 16
  spread over the rest); gate_up with the SiLU gate per checked expert against
  the oracle on the oracle's quantized X and weights (1e-3 and the element
  bound); the quantize of h bit-exact against the oracle's quantize of the
  GPU's h (whole tensor); down per checked expert against the oracle on the
  oracle's quantize of the GPU's h; the combine against the oracle's combine of
  the GPU's y and routing weights (and bit-exact against its stated float32
  slot order rounded to bf16).  Both storage types of h and y (bf16, as
  the benchmark runs, and float32).  With float32 h, the gate_up's fused NVFP4
  epilogue (static global scale) is checked bit-exact as well.

Sources: two-level scaling page (Qwen3.8-Flash-Next-NVFP4), section "Core:
the W4A4 two-level scaling mechanism" (levels 1 and 2) and section "Why only
routed experts" (top-10 of 512 routed experts, fused gate_up / down); QAD
tutorial (Qwen3.6-35B-A3B), section "Why W4A4 rather than W4A16" (W4A4 GEMM,
lm_head included).
"""

import time

import numpy as np
import pytest
import torch

import oracle_pool as OP
from oracle import moe as OM
from oracle import nvfp4 as Q
from oracle import qdq as OD
from moe_nvfp4_quantize_amd import workloads as W

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def B():
    from moe_nvfp4_quantize_amd import nvfp4
    nvfp4.load_library()
    yield nvfp4
    OP.shutdown()


def _host(t):
    return t.detach().float().cpu().numpy()


def _np(t):
    return t.detach().cpu().numpy()


def _log(msg, t0=None):
    extra = f" ({time.time() - t0:.1f} s)" if t0 is not None else ""
    print(f"[configs] {msg}{extra}", flush=True)


def _quantize_exact(B, x, label):
    """GPU dynamic quantize of x, bit-exact against the oracle over the whole
    tensor; returns (GPU (q, s, g), the oracle's (q, s, g))."""
    t0 = time.time()
    gq = B.nvfp4_quantize(x)
    torch.cuda.synchronize()
    xh = _host(x)
    g = Q.global_scale(xh)
    assert gq[2].item() == g, label
    rq, rs = OP.quantize_rows(xh, g)
    np.testing.assert_array_equal(_np(gq[1]), rs, err_msg=label)
    np.testing.assert_array_equal(_np(gq[0]), rq, err_msg=label)
    _log(f"{label} {tuple(x.shape)}: codes, scales, global scale bit-exact", t0)
    return gq, (rq, rs, g)


def _assert_stats(st, label):
    _log(f"{label}: {st['n']:,} outputs, rel_fro {st['rel_fro']:.3e} (vs raw float64 "
         f"{st['rel_fro_raw']:.3e}), element bound max ratio {st['max_ratio']:.3f}, outside {st['bad']}")
    assert st["finite"], label
    assert st["bad"] == 0, (label, st["bad"], st["max_ratio"])
    assert st["rel_fro"] <= TOL, (label, st["rel_fro"])


def _gemm_full(B, a_gpu, b_gpu, a_ref, b_ref, rows_blk, cols_blk, label):
    t0 = time.time()
    y = B.nvfp4_gemm(a_gpu, b_gpu, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yh = _host(y)
    M, N = yh.shape
    tasks = []
    for r in range(0, M, rows_blk):
        for c in range(0, N, cols_blk):
            a = (a_ref[0][r:r + rows_blk], a_ref[1][r:r + rows_blk], a_ref[2])
            b = (b_ref[0][c:c + cols_blk], b_ref[1][c:c + cols_blk], b_ref[2])
            tasks.append((a, b, np.ascontiguousarray(yh[r:r + rows_blk, c:c + cols_blk]), True))
    st = OP.merge(OP.run(OP.gemm_block_check, tasks))
    _assert_stats(st, label)
    _log(f"{label} checked", t0)


def test_prefill_8192x5120_full(B):
    x, w = W.linear_inputs("prefill_8192x5120", device="cuda")
    xg, xr = _quantize_exact(B, x, "prefill X")
    wg, wr = _quantize_exact(B, w, "prefill W")
    del x, w
    _gemm_full(B, xg, wg, xr, wr, 1024, 3200, "prefill GEMM 8192x25600x5120 bf16")


def test_lmhead_128x151936_full(B):
    x, w = W.linear_inputs("lmhead_128x151936", device="cuda")
    xg, xr = _quantize_exact(B, x, "lm_head X")
    wg, wr = _quantize_exact(B, w, "lm_head W")
    del x, w
    _gemm_full(B, xg, wg, xr, wr, 128, 9496, "lm_head GEMM 128x151936x2048 bf16")


# The single-read (register-resident) dynamic quantize holds at most one
# workgroup per compute unit, 512 threads each, 20 bf16 or 10 float32 blocks per
# thread; one block more takes the two-pass path.  Its workspace's first word
# is the parity the single-read kernel flips on every call, so a test sees
# which path ran.
@pytest.mark.parametrize("case", ["bf16 at capacity", "bf16 one row past", "f32 at capacity",
                                  "f32 one row past", "f32 32768x768"])
def test_quantize_single_read_capacity(B, case):
    bf16 = case.startswith("bf16")
    cols = 5120 if bf16 else 1024
    cus = min(torch.cuda.get_device_properties(0).multi_processor_count, 1024)
    cap_rows = cus * 512 * (20 if bf16 else 10) * 16 // cols
    rows = {"at capacity": cap_rows, "one row past": cap_rows + 1}.get(case.split(" ", 1)[1], 32768)
    if case == "f32 32768x768":
        cols = 768
    single_read = rows * cols // 16 <= cus * 512 * (20 if bf16 else 10)
    x = W.random_matrix(rows, cols, seed=rows + cols, dtype=torch.bfloat16 if bf16 else torch.float32,
                        device="cuda")
    t0 = time.time()
    B.nvfp4_quantize(x)  # the stream's workspace has its final size before its parity is read
    torch.cuda.synchronize()
    ws = B._QWS[(torch.cuda.current_device(), int(torch.cuda.current_stream().cuda_stream))]
    before = int(ws[0:4].view(torch.int32).item())
    q, s, g = B.nvfp4_quantize(x)
    torch.cuda.synchronize()
    flipped = int(ws[0:4].view(torch.int32).item()) != before
    assert flipped == single_read, (case, rows, cols, flipped)
    xh = _host(x)
    rg = Q.global_scale(xh)
    assert g.item() == rg
    rq, rs = OP.quantize_rows(xh, rg)
    np.testing.assert_array_equal(_np(s), rs)
    np.testing.assert_array_equal(_np(q), rq)
    _log(f"quantize {case} ({rows}x{cols}): {'single-read' if single_read else 'two-pass'} path, "
         f"codes, scales, global scale bit-exact", t0)


@pytest.mark.parametrize("g_div", [1.0, 64.0])
def test_static_quantize_prefill_full(B, g_div):
    """Static-scale quantize of the whole prefill X (8192x5120 bf16) under a
    calibrated global scale: the tensor's own amax/2688, and that scale / 64
    (blocks whose scale saturates at 448, codes at 6): codes and scales
    bit-exact against the oracle."""
    x, _ = W.linear_inputs("prefill_8192x5120", device="cuda")
    t0 = time.time()
    xh = _host(x)
    g = np.float32(Q.global_scale(xh) / np.float32(g_div))
    q, s, gg = B.nvfp4_quantize(x, g=torch.tensor([float(g)], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert gg.item() == g
    rq, rs = OP.quantize_rows(xh, g)
    np.testing.assert_array_equal(_np(s), rs)
    np.testing.assert_array_equal(_np(q), rq)
    _log(f"static quantize prefill X, g = amax/2688/{g_div:g}: codes and scales bit-exact, "
         f"{int((rs == 0x7E).sum()):,} blocks at scale 448", t0)


@pytest.mark.parametrize("which", ["X", "W"])
def test_qdq_prefill_full(B, which):
    """Quantize-dequantize of the whole prefill X (8192x5120, the single-read
    path) and W (25600x5120, beyond the register capacity: the two-pass path),
    bf16 values and global scale bit-exact against the oracle."""
    x, w = W.linear_inputs("prefill_8192x5120", device="cuda")
    t = x if which == "X" else w
    del x, w
    t0 = time.time()
    y, g = B.nvfp4_qdq(t)
    torch.cuda.synchronize()
    th = _host(t)
    rg = Q.global_scale(th)
    assert g.item() == rg
    ref = OP.qdq_rows(th, rg, "bf16")
    np.testing.assert_array_equal(_host(y), ref)
    _log(f"QDQ prefill {which} {tuple(t.shape)}: every value bit-exact", t0)


@pytest.mark.parametrize("name", ["prefill_8192x5120", "lmhead_128x151936"])
def test_four_over_six_weights_full(B, name):
    """Four-over-six offline quantize of the whole weight matrix of the prefill
    (25600x5120) and lm_head (151936x2048) workloads: codes, block scales and
    global scale bit-exact against the oracle."""
    _, w = W.linear_inputs(name, device="cuda")
    t0 = time.time()
    q, s, g = B.nvfp4_quantize_4over6(w)
    torch.cuda.synchronize()
    wh = _host(w)
    rg = Q.global_scale(wh)
    assert g.item() == rg
    rq, rs, took4 = OP.four_over_six_rows(wh, rg)
    np.testing.assert_array_equal(_np(s), rs)
    np.testing.assert_array_equal(_np(q), rq)
    _log(f"four-over-six {name} W {tuple(w.shape)}: codes, scales, global scale bit-exact; "
         f"{took4 / rs.size:.1%} of blocks take the scale of 4", t0)


def test_fp8_prefill_8192x5120_full(B):
    """FP8 W8A8 on the prefill workload, every element: the GPU's E4M3 codes and
    per-tensor scales of X and W bit-exact against the oracle's over the whole
    tensors, and the whole bf16 GEMM output against the oracle's float64 product
    of those operands (relative Frobenius error and the element bound of
    oracle_pool.fp8_gemm_block_check)."""
    from oracle import fp8 as P
    x, w = W.linear_inputs("prefill_8192x5120", device="cuda")
    gpu, ref = [], []
    for t, label in ((x, "X"), (w, "W")):
        t0 = time.time()
        q, g = B.nvfp4_fp8_quantize(t)
        torch.cuda.synchronize()
        th = _host(t)
        gr = P.scale(th)
        assert g.item() == gr, label
        rq = OP.fp8_encode_rows(th, gr)
        np.testing.assert_array_equal(_np(q), rq, err_msg=label)
        _log(f"FP8 prefill {label} {tuple(t.shape)}: codes and scale bit-exact", t0)
        gpu.append((q, g))
        ref.append((rq, gr))
        del th
    del x, w
    t0 = time.time()
    y = B.nvfp4_fp8_gemm(gpu[0], gpu[1], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yh = _host(y)
    M, N = yh.shape
    tasks = [((ref[0][0][r:r + 1024], ref[0][1]), (ref[1][0][c:c + 3200], ref[1][1]),
              np.ascontiguousarray(yh[r:r + 1024, c:c + 3200]), True)
             for r in range(0, M, 1024) for c in range(0, N, 3200)]
    _assert_stats(OP.merge(OP.run(OP.fp8_gemm_block_check, tasks)), "FP8 prefill GEMM 8192x25600x5120 bf16")
    _log("FP8 prefill GEMM checked", t0)


# ----------------------------------------------------------------------- MoE


def _checked_experts(counts, name):
    E = len(counts)
    if name == "moe_e128_top8":
        return list(range(E))
    order = np.argsort(-counts, kind="stable")
    hot = list(order[:16])
    rest = order[16:]
    spread = list(rest[np.linspace(0, len(rest) - 1, 16).round().astype(int)])
    return sorted(int(e) for e in hot + spread)


def _oracle_experts(stack, experts):
    """The oracle's quantized expert matrices (one global scale each) of the
    checked experts, one pool task per expert; {e: (q, s, g)}."""
    tasks, gs = [], []
    for e in experts:
        we = _host(stack[e])
        gs.append(Q.global_scale(we))
        tasks.append((we, gs[-1]))
    res = OP.run(OP._quantize_chunk, tasks)
    return {e: (q, s, g) for e, (q, s), g in zip(experts, res, gs)}


_MOE = {}


def _moe_setup(B, name):
    """Inputs, offline weights and the stages up to the quantized X, checked
    once per workload and shared by the two storage-type tests."""
    if name in _MOE:
        return _MOE[name]
    _MOE.clear()
    torch.cuda.empty_cache()
    t0 = time.time()
    cfg = W.WORKLOADS[name]
    inp = W.moe_inputs(name, device="cuda")
    k = inp["k"]
    wgu = B.nvfp4_quantize_batched(inp["w_gate_up"])
    wd = B.nvfp4_quantize_batched(inp["w_down"])
    torch.cuda.synchronize()
    _log(f"{name}: inputs drawn and experts quantized on the GPU", t0)

    # routing, bit-exact (weights to 1e-6)
    t0 = time.time()
    r = B.nvfp4_moe_route(inp["logits"], k)
    torch.cuda.synchronize()
    lh = _np(inp["logits"])
    ids, w = OM.route(lh, k)
    offsets, src_row, inv = OM.permute(ids, cfg["E"])
    np.testing.assert_array_equal(_np(r["topk_ids"]), ids)
    np.testing.assert_allclose(_np(r["topk_w"]), w, rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(_np(r["offsets"]), offsets)
    np.testing.assert_array_equal(_np(r["src_row"]), src_row)
    np.testing.assert_array_equal(_np(r["inv"]), inv)
    _log(f"{name}: routing bit-exact", t0)

    # X, bit-exact over the whole tensor
    xg, xr = _quantize_exact(B, inp["x"], f"{name} X")

    # offline expert weights of the checked experts, bit-exact
    t0 = time.time()
    counts = np.diff(offsets)
    experts = _checked_experts(counts, name)
    ogu = _oracle_experts(inp["w_gate_up"], experts)
    od = _oracle_experts(inp["w_down"], experts)
    for e in experts:
        for got, ref in zip((wgu[0][e], wgu[1][e], wgu[2][e]), ogu[e]):
            np.testing.assert_array_equal(_np(got), ref, err_msg=f"gate_up expert {e}")
        for got, ref in zip((wd[0][e], wd[1][e], wd[2][e]), od[e]):
            np.testing.assert_array_equal(_np(got), ref, err_msg=f"down expert {e}")
    _log(f"{name}: offline weights of {len(experts)} experts bit-exact "
         f"(rows per checked expert {counts[experts].min()}..{counts[experts].max()})", t0)
    del inp["w_gate_up"], inp["w_down"]
    torch.cuda.empty_cache()
    st = dict(cfg=cfg, k=k, r=r, xg=xg, xr=xr, wgu=wgu, wd=wd, ogu=ogu, od=od, experts=experts,
              offsets=offsets.astype(np.int64), src_row=src_row, inv=inv)
    _MOE[name] = st
    return st


@pytest.mark.parametrize("inter", ["bf16", "f32"])
@pytest.mark.parametrize("name", ["moe_e128_top8", "moe_e512_top10"])
def test_moe_stagewise(B, name, inter):
    st = _moe_setup(B, name)
    cfg, k, r = st["cfg"], st["k"], st["r"]
    T, H, I = cfg["T"], cfg["H"], cfg["I"]
    R = T * k
    dt = torch.bfloat16 if inter == "bf16" else torch.float32
    is_bf16 = inter == "bf16"
    offsets, experts = st["offsets"], st["experts"]

    # gate_up with the SiLU gate, per checked expert
    t0 = time.time()
    h = B.nvfp4_moe_grouped_gemm(st["xg"], r["src_row"], r["offsets"], R, st["wgu"],
                                 epilogue=B.NVFP4_EPI_SILU_GATE, out_dtype=dt)
    torch.cuda.synchronize()
    hh = _host(h)
    xq, xs, xgs = st["xr"]
    tasks = []
    for e in experts:
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        rows = st["src_row"][lo:hi]
        tasks.append(((xq[rows], xs[rows], xgs), st["ogu"][e], hh[lo:hi], is_bf16))
    _assert_stats(OP.merge(OP.run(OP.silu_gate_block_check, tasks)),
                  f"{name} {inter}: gate_up + SiLU gate, {len(tasks)} experts")
    _log("gate_up checked", t0)

    # quantize of h: bit-exact against the oracle's quantize of the GPU's h
    hg, hr = _quantize_exact(B, h, f"{name} {inter}: h")

    # down, per checked expert, on the oracle's quantize of the GPU's h
    t0 = time.time()
    y = B.nvfp4_moe_grouped_gemm(hg, None, r["offsets"], R, st["wd"], out_dtype=dt)
    torch.cuda.synchronize()
    yh = _host(y)
    tasks = []
    for e in experts:
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        tasks.append(((hr[0][lo:hi], hr[1][lo:hi], hr[2]), st["od"][e], yh[lo:hi], is_bf16))
    _assert_stats(OP.merge(OP.run(OP.gemm_block_check, tasks)),
                  f"{name} {inter}: down, {len(tasks)} experts")
    _log("down checked", t0)

    # combine of the GPU's y with the GPU's routing weights
    t0 = time.time()
    out = B.nvfp4_moe_combine(y, r["topk_w"], r["inv"])
    torch.cuda.synchronize()
    wk = _np(r["topk_w"]).astype(np.float64)
    ref = OM.combine(yh, wk, st["inv"])
    # float32 sum of k products: 2k roundings of at most sum |w y|, then bf16
    mag = np.zeros_like(ref)
    for j in range(k):
        mag += np.abs(wk[:, j:j + 1] * yh[st["inv"][:, j]])
    err = 2 * k * OP.U * mag
    stc = OP.merge([OP._stats(_host(out), ref, err, True)])
    _assert_stats(stc, f"{name} {inter}: combine {T}x{H} bf16")
    # and bit for bit the arithmetic the entry point states: slots in order,
    # each float32 product and addition rounded once, then bf16 (nearest even)
    y32, w32 = yh.astype(np.float32), _np(r["topk_w"])
    acc = np.zeros((T, H), dtype=np.float32)
    for j in range(k):
        acc = acc + w32[:, j:j + 1] * y32[st["inv"][:, j]]
    np.testing.assert_array_equal(_host(out), OD.round_to_bf16(acc))
    _log("combine checked (and bit-exact to its float32 slot order)", t0)

    if inter == "f32":
        # the fused SiLU-gate -> NVFP4 epilogue under a static scale: bit-exact
        # against the oracle's static quantize of the float32 h computed above
        t0 = time.time()
        n = int(offsets[-1])
        g_h = np.float32(Q.global_scale(hh[:n]) / np.float32(2.0))  # saturates some blocks
        hgt = torch.tensor([float(g_h)], dtype=torch.float32, device="cuda")
        fq, fs, _ = B.nvfp4_moe_grouped_gemm_silu_nvfp4(st["xg"], r["src_row"], r["offsets"], R, st["wgu"], hgt)
        torch.cuda.synchronize()
        rq, rs = OP.quantize_rows(hh[:n], g_h)
        np.testing.assert_array_equal(_np(fs[:n]), rs)
        np.testing.assert_array_equal(_np(fq[:n]), rq)
        _log(f"{name}: fused gate_up NVFP4 epilogue bit-exact over {n} rows "
             f"({int((rs == 0x7E).sum())} blocks at scale 448)", t0)
