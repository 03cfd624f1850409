#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the layer over one batch of synthetic, seeded input that is
already resident in HBM:
  dense workloads  : dynamic NVFP4 quantize of the activations (amax pass +
                     encode pass) followed by the W4A4 GEMM against weights
                     quantized once, offline (static), before timing;
  MoE workloads    : router top-k + softmax + permutation, activation quantize,
                     grouped gate_up GEMM with fused SiLU gate, quantize of h,
                     grouped down GEMM, weighted combine.
The default workload is the dense prefill up-projection X[8192x5120] W[25600x5120]
(bf16 in, bf16 out).  ``value`` is the step's effective rate 2*M*N*K / step time
in TFLOP/s; the activation quantizer's HBM rate (GB/s) and each kernel's share of
its roofline are reported beside it.  Kernel durations come from HIP events
recorded on the stream the kernels run on, around each kernel inside the timed
region.

Prints ONE JSON line (see the keys below).
"""

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from moe_nvfp4_quantize_amd import workloads as W  # noqa: E402

METRIC = "NVFP4 GEMM eff. TFLOPS & quantize GB/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 MFMA, TFLOP/s
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense FP4, context only


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # the first ~20 GEMM launches of a process run slower (2.05 ms falling to a
    # steady 1.61 ms for the prefill GEMM) while the clock settles
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="prefill_8192x5120", choices=sorted(W.WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    p.add_argument("--static-scales", action="store_true",
                   help="MoE: static (calibrated) activation scales, h quantized in the gate_up epilogue")
    p.add_argument("--library-reference", action="store_true",
                   help="dense: also time the platform's FP8 (torch._scaled_mm) and bf16 (torch.matmul) "
                        "GEMMs at the same shape, as context")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def profiled_traffic(profile, source):
    """HBM bytes per launch recorded in a committed rocprofv3 summary, or None.

    The summary names the kernel source it was measured on (sha256); when that
    file has changed since, the counters no longer describe it and None is
    returned.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    try:
        fields = {}
        for line in open(path):
            if ":" in line and not line.startswith(("#", " ", "|")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        digest = hashlib.sha256(open(os.path.join(ROOT, source), "rb").read()).hexdigest()
    except OSError:
        return None
    if fields.get("source_sha256") != digest or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def quant_bytes(numel, in_bytes):
    """Algorithmic HBM bytes of one quantize: read x, write codes (0.5 B) and scales (1/16 B)."""
    return numel * (in_bytes + 0.5 + 1.0 / 16.0)


class Timer:
    """Pairs of HIP events on the current stream, averaged over the timed steps."""

    def __init__(self, names):
        self.names = names
        self.ev = {n: [] for n in names}

    def mark(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def add(self, name, start, end):
        self.ev[name].append((start, end))

    def mean_ms(self, name):
        pairs = self.ev[name]
        return sum(a.elapsed_time(b) for a, b in pairs) / max(1, len(pairs))

    def spread_ms(self, name):
        """p10 / median / p90 of the per-step durations (nearest rank)."""
        v = sorted(a.elapsed_time(b) for a, b in self.ev[name])
        if not v:
            return {}
        pick = lambda q: v[min(len(v) - 1, int(q * len(v)))]
        return dict(p10_ms=pick(0.1), median_ms=pick(0.5), p90_ms=pick(0.9))


# ----------------------------------------------------------------- dense


def _time_ms(fn, reps=5):
    """Mean time of back-to-back calls, events around the whole run."""
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def setup_dense(B, name):
    cfg = W.WORKLOADS[name]
    x, w = W.linear_inputs(name, device="cuda")
    wq = B.nvfp4_quantize(w)  # offline static weights, untimed
    # offline weight quantizers, measured beside the step (not part of it)
    offline = dict(plain_ms=_time_ms(lambda: B.nvfp4_quantize(w)),
                   four_over_six_ms=_time_ms(lambda: B.nvfp4_quantize_4over6(w)),
                   elements=w.numel())
    # the same layer in FP8 W8A8 (per-tensor E4M3), weights quantized offline
    w8 = B.nvfp4_fp8_quantize(w)
    del w
    xq = (torch.empty((cfg["M"], cfg["K"] // 2), dtype=torch.uint8, device="cuda"),
          torch.empty((cfg["M"], cfg["K"] // 16), dtype=torch.uint8, device="cuda"),
          torch.empty(1, dtype=torch.float32, device="cuda"))
    out_dtype = torch.bfloat16 if cfg["out"] == "bf16" else torch.float32
    y = torch.empty((cfg["M"], cfg["N"]), dtype=out_dtype, device="cuda")
    # static (calibrated) activation scale: amax of 512 fresh rows / 2688, untimed
    g_static = B.nvfp4_quantize(W.calibration_rows(name, 512, device="cuda"))[2].clone()
    xq_static = (torch.empty_like(xq[0]), torch.empty_like(xq[1]), g_static)
    qdq_ms = _time_ms(lambda: B.nvfp4_qdq(x))
    return dict(cfg=cfg, name=name, x=x, wq=wq, xq=xq, y=y, xq_static=xq_static, offline=offline,
                qdq_ms=qdq_ms, w8=w8)


def measure_fp8(B, st, reps):
    """FP8 W8A8 layer at the same shape: dynamic per-tensor quantize of X, then
    the FP8 GEMM, each timed back to back, and the two as a step."""
    cfg = st["cfg"]
    x8 = (torch.empty((cfg["M"], cfg["K"]), dtype=torch.uint8, device="cuda"),
          torch.empty(1, dtype=torch.float32, device="cuda"))
    q_ms = _time_ms(lambda: B.nvfp4_fp8_quantize(st["x"], out=x8), reps)
    g_ms = _time_ms(lambda: B.nvfp4_fp8_gemm(x8, st["w8"], out=st["y"]), reps)

    def both():
        B.nvfp4_fp8_quantize(st["x"], out=x8)
        B.nvfp4_fp8_gemm(x8, st["w8"], out=st["y"])
    st["fp8"] = dict(quantize_ms=q_ms, gemm_ms=g_ms, step_ms=_time_ms(both, reps))


def step_dense(B, st, timer=None):
    t0 = timer.mark() if timer else None
    B.nvfp4_quantize(st["x"], out=st["xq"])
    t1 = timer.mark() if timer else None
    B.nvfp4_gemm(st["xq"], st["wq"], out=st["y"])
    if timer:
        t2 = timer.mark()
        timer.add("quantize", t0, t1)
        timer.add("gemm", t1, t2)


def library_reference(st, reps):
    """The platform libraries' GEMMs at the dense shape (context, not part of the path):
    FP8 E4M3 x E4M3 with unit scales through torch._scaled_mm, and bf16 x bf16 through
    torch.matmul, on random operands of the workload's shape."""
    cfg = st["cfg"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    flops = 2.0 * M * N * K
    out = {}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    a = torch.randn((M, K), generator=gen, device="cuda")
    b = torch.randn((N, K), generator=gen, device="cuda")
    try:
        a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
        one = torch.ones((), device="cuda")
        ms = _time_ms(lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16), reps)
        out["fp8_scaled_mm"] = dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12)
        del a8, b8
    except Exception as ex:  # the library call is optional context
        out["fp8_scaled_mm"] = dict(error=str(ex)[:200])
    ab, bb = a.to(torch.bfloat16), b.to(torch.bfloat16)
    del a, b
    ms = _time_ms(lambda: ab @ bb.t(), reps)
    out["bf16_matmul"] = dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12)
    out["note"] = "platform GEMM libraries through torch at the same shape; context only"
    st["library_reference"] = out


def report_dense(st, timer, step_ms):
    cfg = st["cfg"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    flops = 2.0 * M * N * K
    gemm_ms = timer.mean_ms("gemm")
    q_ms = timer.mean_ms("quantize")
    in_b = 2 if cfg["x_dtype"] == "bf16" else 4
    out_b = 2 if cfg["out"] == "bf16" else 4
    qbytes = quant_bytes(M * K, in_b)
    gemm_bytes = 0.5625 * (M * K + N * K) + out_b * M * N
    t_mfma = flops / (F16_MFMA_PEAK_TFLOPS * 1e12)
    t_hbm = gemm_bytes / (HBM_PEAK_GBS * 1e9)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    gemm_gbs = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    if t_mfma >= t_hbm:
        roof = dict(bound="mfma", achieved=gemm_tflops, peak=F16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=gemm_tflops / F16_MFMA_PEAK_TFLOPS)
    else:
        roof = dict(bound="hbm", achieved=gemm_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=gemm_gbs / HBM_PEAK_GBS)
    traffic = None
    profile = {"prefill_8192x5120": "gemm_prefill_8192x5120x25600.md",
               "lmhead_128x151936": "gemm_lmhead_128x151936x2048.md"}.get(st["name"])
    if profile:
        traffic = profiled_traffic(profile, "moe_nvfp4_quantize_amd/csrc/gemm.hip")
    kernel = "nvfp4 gemm_dma_kernel" if K % 256 == 0 else "nvfp4 gemm_kernel"
    roof.update(kernel=kernel, traffic=traffic,
                per_launch=dict(flops=flops, algorithmic_bytes=gemm_bytes, avg_ms=gemm_ms))
    q_gbs = qbytes / (q_ms * 1e-3) / 1e9
    extra = dict(
        gemm=dict(avg_ms=gemm_ms, tflops=gemm_tflops, frac_f16_peak=gemm_tflops / F16_MFMA_PEAK_TFLOPS,
                  frac_fp4_peak=gemm_tflops / FP4_MFMA_PEAK_TFLOPS, gbs=gemm_gbs, **timer.spread_ms("gemm")),
        quantize=dict(avg_ms=q_ms, gbs=q_gbs, frac_hbm=q_gbs / HBM_PEAK_GBS,
                      algorithmic_bytes=qbytes, note="in-step interval, after the GEMM",
                      **timer.spread_ms("quantize")),
    )
    if "quantize_iso_ms" in st:
        iso = st["quantize_iso_ms"]
        extra["quantize_back_to_back"] = dict(avg_ms=iso, gbs=qbytes / (iso * 1e-3) / 1e9,
                                              frac_hbm=qbytes / (iso * 1e-3) / 1e9 / HBM_PEAK_GBS)
    if "offline" in st:
        o = st["offline"]
        in_b = 2 if cfg["x_dtype"] == "bf16" else 4
        wbytes = quant_bytes(o["elements"], in_b)
        extra["weights_offline"] = dict(
            plain_ms=o["plain_ms"], plain_gbs=wbytes / (o["plain_ms"] * 1e-3) / 1e9,
            four_over_six_ms=o["four_over_six_ms"],
            four_over_six_gbs=wbytes / (o["four_over_six_ms"] * 1e-3) / 1e9,
            note="one-time weight quantize (two passes over W: amax, encode); "
                 "algorithmic bytes count W once")
    if "qdq_ms" in st:
        in_b = 2 if cfg["x_dtype"] == "bf16" else 4
        qb = 2.0 * in_b * M * K
        extra["qdq"] = dict(avg_ms=st["qdq_ms"], gbs=qb / (st["qdq_ms"] * 1e-3) / 1e9,
                            frac_hbm=qb / (st["qdq_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            note="dynamic quantize-dequantize of X, back to back; bytes: read + write X")
    if "quantize_static_ms" in st:
        sq = st["quantize_static_ms"]
        extra["quantize_static"] = dict(
            avg_ms=sq, gbs=qbytes / (sq * 1e-3) / 1e9, frac_hbm=qbytes / (sq * 1e-3) / 1e9 / HBM_PEAK_GBS,
            note="static global scale calibrated on 512 other rows (amax/2688): one streaming pass; "
                 "timed in the step, after the GEMM")
    if "fp8" in st:
        f = st["fp8"]
        in_b = 2 if cfg["x_dtype"] == "bf16" else 4
        f8_qbytes = (in_b + 1.0) * M * K
        f8_tflops = flops / (f["gemm_ms"] * 1e-3) / 1e12
        f8_traffic = None
        if st["name"] == "prefill_8192x5120":
            f8_traffic = profiled_traffic("fp8_gemm_prefill_8192x5120x25600.md",
                                          "moe_nvfp4_quantize_amd/csrc/fp8_gemm.hip")
        extra["fp8_w8a8"] = dict(
            gemm_ms=f["gemm_ms"], gemm_tflops=f8_tflops, gemm_frac_fp8_peak=f8_tflops / FP8_MFMA_PEAK_TFLOPS,
            gemm_traffic=f8_traffic, gemm_algorithmic_bytes=(M * K + N * K) + out_b * M * N,
            quantize_ms=f["quantize_ms"], quantize_gbs=f8_qbytes / (f["quantize_ms"] * 1e-3) / 1e9,
            quantize_frac_hbm=f8_qbytes / (f["quantize_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            step_ms=f["step_ms"], step_tflops=flops / (f["step_ms"] * 1e-3) / 1e12,
            note="same layer in FP8 E4M3 W8A8 (per-tensor scales; fp8_gemm_dma_kernel on the FP8 MFMA); "
                 "weights quantized offline; each kernel timed back to back; quantize bytes: read X, "
                 "write one byte per element")
    if "library_reference" in st:
        extra["library_reference"] = st["library_reference"]
    value = flops / (step_ms * 1e-3) / 1e12
    config = dict(workload=st["name"], M=M, N=N, K=K, x=cfg["x_dtype"], out=cfg["out"],
                  weights="NVFP4, quantized offline (static)", activations="NVFP4, dynamic, quantized in the step")
    return value, "TFLOP/s", roof, extra, config


# ------------------------------------------------------------------- MoE


def setup_moe(B, name, static=False):
    cfg = W.WORKLOADS[name]
    inp = W.moe_inputs(name, device="cuda")
    wgu = B.nvfp4_quantize_batched(inp["w_gate_up"])
    wd = B.nvfp4_quantize_batched(inp["w_down"])
    del inp["w_gate_up"], inp["w_down"]
    st = dict(cfg=cfg, name=name, x=inp["x"], logits=inp["logits"], k=inp["k"], wgu=wgu, wd=wd,
              static=static)
    if static:
        # calibrate the two activation scales (max over a batch of other tokens), untimed
        T_cal = min(cfg["T"], 2048)
        lg, xc = W.moe_calibration_inputs(name, T_cal, device="cuda")
        r = B.nvfp4_moe_route(lg, inp["k"])
        xq = B.nvfp4_quantize(xc)
        h = B.nvfp4_moe_grouped_gemm(xq, r["src_row"], r["offsets"], T_cal * inp["k"], wgu,
                                     epilogue=B.NVFP4_EPI_SILU_GATE, out_dtype=torch.float32)
        st["gx"] = xq[2].clone()
        st["gh"] = B.nvfp4_quantize(h)[2].clone()
        del h
    return st


def step_moe_static(B, st, timer=None):
    T = st["x"].shape[0]
    k = st["k"]
    R = T * k
    m = [timer.mark()] if timer else None
    r = B.nvfp4_moe_route(st["logits"], k)
    if timer: m.append(timer.mark())
    xq = B.nvfp4_quantize(st["x"], g=st["gx"])
    if timer: m.append(timer.mark())
    hq = B.nvfp4_moe_grouped_gemm_silu_nvfp4(xq, r["src_row"], r["offsets"], R, st["wgu"], st["gh"])
    if timer: m.append(timer.mark())
    y = B.nvfp4_moe_grouped_gemm(hq, None, r["offsets"], R, st["wd"], out_dtype=torch.bfloat16)
    if timer: m.append(timer.mark())
    B.nvfp4_moe_combine(y, r["topk_w"], r["inv"])
    if timer:
        m.append(timer.mark())
        for i, n in enumerate(["route", "quantize_x", "gate_up", "down", "combine"]):
            timer.add(n, m[i], m[i + 1])


def step_moe(B, st, timer=None):
    T = st["x"].shape[0]
    k = st["k"]
    R = T * k
    m = [timer.mark()] if timer else None
    r = B.nvfp4_moe_route(st["logits"], k)
    if timer: m.append(timer.mark())
    xq = B.nvfp4_quantize(st["x"])
    if timer: m.append(timer.mark())
    h = B.nvfp4_moe_grouped_gemm(xq, r["src_row"], r["offsets"], R, st["wgu"],
                                 epilogue=B.NVFP4_EPI_SILU_GATE, out_dtype=torch.bfloat16)
    if timer: m.append(timer.mark())
    hq = B.nvfp4_quantize(h)
    if timer: m.append(timer.mark())
    y = B.nvfp4_moe_grouped_gemm(hq, None, r["offsets"], R, st["wd"], out_dtype=torch.bfloat16)
    if timer: m.append(timer.mark())
    B.nvfp4_moe_combine(y, r["topk_w"], r["inv"])
    if timer:
        m.append(timer.mark())
        for i, n in enumerate(["route", "quantize_x", "gate_up", "quantize_h", "down", "combine"]):
            timer.add(n, m[i], m[i + 1])


def report_moe(st, timer, step_ms):
    cfg = st["cfg"]
    T, E, k, H, I = cfg["T"], cfg["E"], cfg["k"], cfg["H"], cfg["I"]
    R = T * k
    f_gu = 2.0 * R * 2 * I * H
    f_d = 2.0 * R * H * I
    flops = f_gu + f_d
    gu_ms = timer.mean_ms("gate_up")
    gu_tflops = f_gu / (gu_ms * 1e-3) / 1e12
    kernel = "nvfp4 gemm_dma_kernel" if H % 256 == 0 else "nvfp4 gemm_kernel"
    kernel += " (grouped, SiLU gate" + (" -> NVFP4 h)" if st["static"] else ")")
    # HBM bytes of the gate_up launch from the committed summary of the dynamic
    # step (the static step's gate_up writes NVFP4 h instead: not measured)
    traffic = None
    if not st["static"]:
        traffic = profiled_traffic(f"moe_step_{st['name'][len('moe_'):]}.md",
                                   "moe_nvfp4_quantize_amd/csrc/gemm.hip")
    roof = dict(bound="mfma", achieved=gu_tflops, peak=F16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                frac=gu_tflops / F16_MFMA_PEAK_TFLOPS, kernel=kernel, traffic=traffic,
                per_launch=dict(flops=f_gu, avg_ms=gu_ms))
    parts = {n: timer.mean_ms(n) for n in timer.names}
    d_ms = parts["down"]
    extra = dict(stages_ms=parts, stages_spread_ms={n: timer.spread_ms(n) for n in timer.names},
                 down=dict(tflops=f_d / (d_ms * 1e-3) / 1e12))
    if "quantize_h" in parts:
        qh_bytes = quant_bytes(R * I, 2)  # h stored in bf16
        extra["quantize_h"] = dict(gbs=qh_bytes / (parts["quantize_h"] * 1e-3) / 1e9)
    value = flops / (step_ms * 1e-3) / 1e12
    config = dict(workload=st["name"], T=T, E=E, k=k, H=H, I=I, x="bf16", out="bf16",
                  experts="NVFP4 gate_up [2I x H] and down [H x I], quantized offline",
                  intermediates="h and y stored in bf16, combine in float32",
                  activation_scales="static (calibrated on 2048 other tokens), h quantized in the "
                                    "gate_up epilogue" if st["static"] else "dynamic")
    return value, "TFLOP/s", roof, extra, config


# ----------------------------------------------------------- CPU baseline


def cpu_baseline_dense(cfg_name):
    """The oracle on a bounded sample of the dense step, extrapolated to the full step."""
    import numpy as np
    from oracle import gemm as OG
    from oracle import nvfp4 as OQ
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    cfg = W.WORKLOADS[cfg_name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    mq, mg, ng = min(M, 256), min(M, 64), min(N, 2560)
    x, w = W.linear_inputs(cfg_name, device="cpu")
    xh = x.float().numpy()
    wh = w[:ng].float().numpy()
    gw = OQ.global_scale(w.float().numpy())
    wq = OQ.quantize(wh, g=gw)  # offline weights: not timed
    t0 = time.perf_counter()
    gx = OQ.global_scale(xh)
    OQ.quantize(xh[:mq], g=gx)
    tq = time.perf_counter() - t0
    xq = OQ.quantize(xh[:mg], g=gx)
    t0 = time.perf_counter()
    OG.gemm(*xq, *wq)
    tg = time.perf_counter() - t0
    step_s = tq * (M / mq) + tg * (M * N) / (mg * ng)
    return dict(value=2.0 * M * N * K / step_s / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"quantize {mq} of {M} activation rows (global scale over all rows) and GEMM "
                       f"{mg}x{ng} of {M}x{N} outputs (K={K}), float64 numpy; times scaled by the "
                       f"row/output counts to one full step ({step_s:.1f} s)")


def cpu_baseline_moe(cfg_name):
    return None


# ------------------------------------------------------------------- main


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    from moe_nvfp4_quantize_amd import nvfp4 as B
    B.load_library()
    torch.cuda.set_device(0)
    kind = W.WORKLOADS[args.workload]["kind"]
    if kind == "linear":
        st, step, report = setup_dense(B, args.workload), step_dense, report_dense
        names = ["quantize", "gemm"]
    else:
        st, report = setup_moe(B, args.workload, static=args.static_scales), report_moe
        if args.static_scales:
            step, names = step_moe_static, ["route", "quantize_x", "gate_up", "down", "combine"]
        else:
            step, names = step_moe, ["route", "quantize_x", "gate_up", "quantize_h", "down", "combine"]

    for _ in range(args.warmup):
        step(B, st)
    torch.cuda.synchronize()

    # whole-step wall time: K steps between two synchronizations
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step(B, st)
    t_end.record()
    torch.cuda.synchronize()
    step_ms = t_start.elapsed_time(t_end) / args.steps

    # per-kernel durations: the same steps again with events around every kernel
    timer = Timer(names)
    for _ in range(args.steps):
        step(B, st, timer)
    torch.cuda.synchronize()

    if kind == "linear":
        # the activation quantizer alone, back to back (no GEMM in between)
        for _ in range(3):
            B.nvfp4_quantize(st["x"], out=st["xq"])
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record()
        for _ in range(args.steps):
            B.nvfp4_quantize(st["x"], out=st["xq"])
        q1.record()
        torch.cuda.synchronize()
        st["quantize_iso_ms"] = q0.elapsed_time(q1) / args.steps
        # the static-scale quantizer where it would sit in a step: after a GEMM
        sq = []
        for _ in range(args.steps):
            B.nvfp4_gemm(st["xq"], st["wq"], out=st["y"])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.nvfp4_quantize(st["x"], g=st["xq_static"][2], out=st["xq_static"])
            e1.record()
            sq.append((e0, e1))
        torch.cuda.synchronize()
        st["quantize_static_ms"] = sum(a.elapsed_time(b) for a, b in sq) / len(sq)

    if kind == "linear":
        measure_fp8(B, st, args.steps)
        if args.library_reference:
            library_reference(st, args.steps)

    if args.copy_probe_mib:
        a = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    value, unit, roof, extra, config = report(st, timer, step_ms)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_dense(args.workload) if kind == "linear" else cpu_baseline_moe(args.workload)
    line = dict(metric=METRIC, value=value, unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=step_ms, higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="f16", data="synthetic", config=config, roofline=roof, cpu_baseline=cpu,
                **extra)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
