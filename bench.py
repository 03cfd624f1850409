#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--iters N]
                    [--configs LIST|all|none] [--no-cpu-baseline]

A step is one pass of the layer over one batch of synthetic, seeded input that
is already resident in HBM:
  dense workloads : dynamic NVFP4 quantize of the activations followed by the
                    W4A4 GEMM against weights quantized once, offline (static),
                    before timing;
  MoE workloads   : router top-k + softmax + permutation, activation quantize,
                    grouped gate_up GEMM with the SiLU gate, quantize of h,
                    grouped down GEMM, weighted combine.
The headline workload (default: the dense prefill up-projection X[8192x5120]
W[25600x5120], bf16 in and out) is timed for exactly K steps after W warm-up
steps; ``value`` is its effective rate 2*M*N*K / step time in TFLOP/s.  The
other large workloads (lm_head, both MoE layers) are measured in the same run
under ``configs``, over --iters steps each.

Cold caches: every step reads its inputs from one of several copies, rotated
so that the copies in turn exceed 512 MB (twice the Infinity Cache): no step
finds its inputs in the caches because an earlier step read them.

Kernel durations come from HIP events recorded on the stream the kernels run
on: around each kernel for the per-kernel figures (median, p10, p90, mean of
--iters launches), and around a whole run of launches for the back-to-back
rates (no event between launches).  ``roofline`` is the dominant kernel of the
headline workload against the MI355X peak of its bound; ``traffic`` is its HBM
bytes per launch from the committed rocprofv3 counter summary, if that was
taken on the current kernel source.  ``ceilings`` are two streaming kernels
(libnvfp4_ceiling.so) with the quantizer's read, and read-plus-write, traffic:
the HBM rate this GPU delivers to such a kernel.  ``cpu_baseline`` is the
oracle (CPU reference) timed on this host: 3 repeats (median), one core and
all cores, on a bounded sample scaled to one step.

Prints ONE JSON line.
"""

import argparse
import contextlib
import gc
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from moe_nvfp4_quantize_amd import workloads as W  # noqa: E402

METRIC = "NVFP4 GEMM eff. TFLOPS & quantize GB/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 MFMA, TFLOP/s
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense FP4, context only
ROTATE_BYTES = 512 << 20       # rotated input copies exceed this, twice the Infinity Cache
LARGE = ["prefill_8192x5120", "lmhead_128x151936", "moe_e128_top8", "moe_e512_top10"]
PROFILES = {"prefill_8192x5120": "gemm_prefill_8192x5120x25600.md",
            "lmhead_128x151936": "gemm_lmhead_128x151936x2048.md",
            "moe_e128_top8": "moe_step_e128_top8.md",
            "moe_e512_top10": "moe_step_e512_top10.md"}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="prefill_8192x5120", choices=sorted(W.WORKLOADS))
    p.add_argument("--iters", type=int, default=100,
                   help="timed iterations of the per-kernel figures and of the other workloads")
    p.add_argument("--configs", default="all",
                   help="other workloads measured under 'configs': comma list, 'all' (default) or 'none'")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing legs")
    p.add_argument("--static-scales", action="store_true",
                   help="MoE headline: static (calibrated) activation scales, h quantized in the gate_up epilogue")
    p.add_argument("--library-reference", action="store_true",
                   help="dense: also time the platform's FP8 (torch._scaled_mm) and bf16 (torch.matmul) "
                        "GEMMs at the same shape, as context")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def profiled_traffic(profile, source, key="traffic_bytes_per_launch"):
    """HBM bytes per launch recorded in a committed rocprofv3 summary, or None.

    The summary names the kernel source it was measured on (sha256); when that
    file has changed since, the counters no longer describe it and None is
    returned.
    """
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
    if fields.get("source_sha256") != digest or key not in fields:
        return None
    return int(fields[key])


def quant_bytes(numel, in_bytes):
    """Algorithmic HBM bytes of one quantize: read x, write codes (0.5 B) and scales (1/16 B)."""
    return numel * (in_bytes + 0.5 + 1.0 / 16.0)


def n_copies(nbytes):
    """Copies of an input of nbytes that together exceed ROTATE_BYTES."""
    return ROTATE_BYTES // max(1, int(nbytes)) + 1


def tensor_bytes(ts):
    return sum(t.numel() * t.element_size() for t in ts)


def spread(vals):
    """p10 / median / p90 / mean of a list of durations (ms), nearest rank."""
    v = sorted(vals)
    if not v:
        return {}
    pick = lambda q: v[min(len(v) - 1, int(q * len(v)))]
    return dict(p10_ms=pick(0.1), median_ms=statistics.median(v), p90_ms=pick(0.9), mean_ms=sum(v) / len(v),
                n=len(v))


class Timer:
    """Pairs of HIP events on the current stream (the stream the kernels run on)."""

    def __init__(self, names):
        self.names = names
        self.ev = {n: [] for n in names}

    def mark(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def add(self, name, start, end):
        self.ev[name].append((start, end))

    def durations(self, name):
        return [a.elapsed_time(b) for a, b in self.ev[name]]

    def stats(self):
        return {n: spread(self.durations(n)) for n in self.names}


@contextlib.contextmanager
def gc_paused():
    """Python's collector paused (after a collection) while a timed loop runs:
    a collection between the two events around a kernel would leave the GPU
    idle inside the interval, waiting for the next launch."""
    gc.collect()
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


def run_timed(step, n, first=0):
    """Mean ms of n steps (step(i)) with events around the whole run."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with gc_paused():
        a.record()
        for i in range(first, first + n):
            step(i)
        b.record()
        torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def run_kernels(step, names, n, first=0):
    """Per-kernel event durations over n steps (step(i, timer))."""
    tm = Timer(names)
    with gc_paused():
        for i in range(first, first + n):
            step(i, tm)
        torch.cuda.synchronize()
    return tm.stats()


def roofline_entry(flops, nbytes, ms, kernel, traffic, peak_tflops=F16_MFMA_PEAK_TFLOPS):
    """Roofline of one kernel: bound by whichever of MFMA time and HBM time is
    longer at peak; the fraction is that time over the measured one."""
    t_mfma = flops / (peak_tflops * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    s = ms * 1e-3
    if t_mfma >= t_hbm:
        ach = flops / s / 1e12
        r = dict(bound="mfma", achieved=ach, peak=peak_tflops, unit="TFLOP/s", frac=ach / peak_tflops)
    else:
        ach = nbytes / s / 1e9
        r = dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s", frac=ach / HBM_PEAK_GBS)
    r.update(traffic=traffic, kernel=kernel,
             per_launch=dict(flops=flops, algorithmic_bytes=nbytes, avg_ms=ms,
                             frac_of_max_roof=max(t_mfma, t_hbm) / s))
    return r


# ------------------------------------------------------------------ dense


def dense_setup(B, name):
    cfg = W.WORKLOADS[name]
    x, w = W.linear_inputs(name, device="cuda")
    wq = B.nvfp4_quantize(w)  # offline static weights, untimed
    st = dict(cfg=cfg, name=name, w=w)
    st["xs"] = [x] + [x.clone() for _ in range(n_copies(tensor_bytes([x])) - 1)]
    st["wqs"] = [wq] + [tuple(t.clone() for t in wq) for _ in range(n_copies(tensor_bytes(wq)) - 1)]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    st["xq"] = (torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                torch.empty((M, K // 16), dtype=torch.uint8, device="cuda"),
                torch.empty(1, dtype=torch.float32, device="cuda"))
    out_dtype = torch.bfloat16 if cfg["out"] == "bf16" else torch.float32
    st["y"] = torch.empty((M, N), dtype=out_dtype, device="cuda")
    return st


def dense_step(B, st):
    xs, wqs, xq, y = st["xs"], st["wqs"], st["xq"], st["y"]

    def step(i, tm=None):
        t0 = tm.mark() if tm else None
        B.nvfp4_quantize(xs[i % len(xs)], out=xq)
        t1 = tm.mark() if tm else None
        B.nvfp4_gemm(xq, wqs[i % len(wqs)], out=y)
        if tm:
            t2 = tm.mark()
            tm.add("quantize", t0, t1)
            tm.add("gemm", t1, t2)
    return step, ["quantize", "gemm"]


def dense_report(st, step_ms, kstats, steps):
    cfg = st["cfg"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    flops = 2.0 * M * N * K
    out_b = 2 if cfg["out"] == "bf16" else 4
    in_b = 2 if cfg["x_dtype"] == "bf16" else 4
    gemm_bytes = 0.5625 * (M * K + N * K) + out_b * M * N
    g = kstats["gemm"]
    traffic = profiled_traffic(PROFILES[st["name"]], "moe_nvfp4_quantize_amd/csrc/gemm.hip") \
        if st["name"] in PROFILES else None
    roof = roofline_entry(flops, gemm_bytes, g["mean_ms"], "nvfp4 gemm_dma_kernel" if K % 256 == 0
                          else "nvfp4 gemm_kernel", traffic)
    qb = quant_bytes(M * K, in_b)
    out = dict(ms_per_step=step_ms, value=flops / (step_ms * 1e-3) / 1e12, unit="TFLOP/s", steps=steps,
               roofline=roof,
               kernels=dict(gemm=dict(g, tflops=flops / (g["mean_ms"] * 1e-3) / 1e12,
                                      frac_f16_peak=flops / (g["mean_ms"] * 1e-3) / 1e12 / F16_MFMA_PEAK_TFLOPS,
                                      frac_fp4_peak=flops / (g["mean_ms"] * 1e-3) / 1e12 / FP4_MFMA_PEAK_TFLOPS),
                            quantize=dict(kstats["quantize"], algorithmic_bytes=qb,
                                          note="per-launch events (each pair adds a few us to a kernel "
                                               "this short)")),
               config=dict(workload=st["name"], M=M, N=N, K=K, x=cfg["x_dtype"], out=cfg["out"],
                           weights="NVFP4, quantized offline (static)",
                           activations="NVFP4, dynamic, quantized in the step",
                           rotation=dict(x_copies=len(st["xs"]), weight_copies=len(st["wqs"]))))
    return out


def quantizer_legs(B, st, iters):
    """The activation quantizer cold and back to back (events around the whole
    run of launches over the rotating copies of X), the static-scale pass, the
    offline weight quantizers, quantize-dequantize and the FP8 W8A8 layer."""
    cfg = st["cfg"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    in_b = 2 if cfg["x_dtype"] == "bf16" else 4
    xs, xq = st["xs"], st["xq"]
    qb = quant_bytes(M * K, in_b)
    res = {}
    runs = [run_timed(lambda i: B.nvfp4_quantize(xs[i % len(xs)], out=xq), iters) for _ in range(3)]
    ms = statistics.median(runs)
    res["quantize_cold"] = dict(ms=ms, runs_ms=runs, gbs=qb / (ms * 1e-3) / 1e9,
                                frac_hbm=qb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, algorithmic_bytes=qb,
                                note=f"dynamic; {iters} launches back to back over {len(xs)} copies of X, "
                                     "events around the run (median of 3 runs)")
    # static (calibrated) scale: one streaming pass
    g_static = B.nvfp4_quantize(W.calibration_rows(st["name"], 512, device="cuda"))[2].clone()
    xq_s = (torch.empty_like(xq[0]), torch.empty_like(xq[1]), g_static)
    ms = statistics.median([run_timed(lambda i: B.nvfp4_quantize(xs[i % len(xs)], g=g_static, out=xq_s), iters)
                            for _ in range(3)])
    res["quantize_static_cold"] = dict(ms=ms, gbs=qb / (ms * 1e-3) / 1e9,
                                       frac_hbm=qb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       note="global scale calibrated on 512 other rows (amax/2688): one "
                                            "streaming pass; back to back over the copies of X")
    # allocation-free entry point, same work
    ms = run_timed(lambda i: B.nvfp4_quantize_noalloc(xs[i % len(xs)], out=xq), iters)
    res["quantize_noalloc_cold"] = dict(ms=ms, gbs=qb / (ms * 1e-3) / 1e9)
    # offline weights: plain and four-over-six (two passes over W)
    w = st["w"]
    wb = quant_bytes(w.numel(), in_b)
    reps = max(5, iters // 10)
    pm = run_timed(lambda i: B.nvfp4_quantize(w), reps)
    fm = run_timed(lambda i: B.nvfp4_quantize_4over6(w), reps)
    res["weights_offline"] = dict(plain_ms=pm, plain_gbs=wb / (pm * 1e-3) / 1e9, four_over_six_ms=fm,
                                  four_over_six_gbs=wb / (fm * 1e-3) / 1e9,
                                  note="one-time weight quantize (amax pass, encode pass); algorithmic bytes "
                                       "count W once")
    # quantize-dequantize of X (the QAD forward), dynamic
    ys = torch.empty_like(xs[0])
    ms = run_timed(lambda i: B.nvfp4_qdq(xs[i % len(xs)], out=ys), iters)
    qdb = 2.0 * in_b * M * K
    res["qdq_cold"] = dict(ms=ms, gbs=qdb / (ms * 1e-3) / 1e9, frac_hbm=qdb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           note="dynamic; bytes: read + write X")
    # FP8 W8A8 at the same shape (per-tensor E4M3), weights quantized offline
    w8 = B.nvfp4_fp8_quantize(w)
    x8 = (torch.empty((M, K), dtype=torch.uint8, device="cuda"), torch.empty(1, dtype=torch.float32, device="cuda"))
    q8 = run_timed(lambda i: B.nvfp4_fp8_quantize(xs[i % len(xs)], out=x8), iters)
    g8 = run_timed(lambda i: B.nvfp4_fp8_gemm(x8, w8, out=st["y"]), max(20, iters // 5))
    flops = 2.0 * M * N * K
    out_b = 2 if cfg["out"] == "bf16" else 4
    f8_traffic = profiled_traffic("fp8_gemm_prefill_8192x5120x25600.md", "moe_nvfp4_quantize_amd/csrc/fp8_gemm.hip") \
        if st["name"] == "prefill_8192x5120" else None
    res["fp8_w8a8"] = dict(gemm_ms=g8, gemm_tflops=flops / (g8 * 1e-3) / 1e12,
                           gemm_frac_fp8_peak=flops / (g8 * 1e-3) / 1e12 / FP8_MFMA_PEAK_TFLOPS,
                           gemm_traffic=f8_traffic, gemm_algorithmic_bytes=(M * K + N * K) + out_b * M * N,
                           quantize_ms=q8, quantize_gbs=(in_b + 1.0) * M * K / (q8 * 1e-3) / 1e9,
                           note="same layer in FP8 E4M3 W8A8 (per-tensor scales) on the FP8 MFMA; weights "
                                "quantized offline; each kernel back to back")
    del w8, x8, ys
    return res


def ceilings(st, iters):
    """HBM rates of the two ceiling kernels over the rotating copies of X:
    read only, and read plus the quantizer's writes (into the quantizer's own
    output buffers); best of 1, 2 and 4 workgroups per compute unit."""
    path = os.path.join(ROOT, "moe_nvfp4_quantize_amd", "libnvfp4_ceiling.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.ceiling_grid.restype = ctypes.c_uint32
    lib.ceiling_grid.argtypes = [ctypes.c_uint32]
    for fn in (lib.ceiling_read, lib.ceiling_read_write):
        fn.restype = ctypes.c_int
    lib.ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    lib.ceiling_read_write.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_uint32, ctypes.c_void_p]
    xs, xq = st["xs"], st["xq"]
    nbytes = xs[0].numel() * xs[0].element_size()
    sink = torch.empty(lib.ceiling_grid(4), dtype=torch.int32, device="cuda")
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    for label, total, call in (
            ("read", nbytes, lambda x, wpc: lib.ceiling_read(x.data_ptr(), nbytes, sink.data_ptr(), wpc, stream())),
            ("read_write", nbytes * (1 + 0.25 + 1 / 32),
             lambda x, wpc: lib.ceiling_read_write(x.data_ptr(), nbytes, xq[0].data_ptr(), xq[1].data_ptr(), wpc,
                                                   stream()))):
        best = None
        for wpc in (1, 2, 4):
            if call(xs[0], wpc) != 0:
                return None
            ms = statistics.median([run_timed(lambda i: call(xs[i % len(xs)], wpc), iters) for _ in range(3)])
            gbs = total / (ms * 1e-3) / 1e9
            if best is None or gbs > best["gbs"]:
                best = dict(gbs=gbs, ms=ms, wgs_per_cu=wpc, frac_hbm=gbs / HBM_PEAK_GBS, bytes=total)
        out[label] = best
    out["note"] = ("streaming kernels with the quantizer's access pattern over the same rotating copies of X: "
                   "read 32 B per 16 bf16 elements (read) and also write 8 B + 1 B to its code and scale "
                   "arrays (read_write); best of 1, 2, 4 workgroups per CU")
    return out


def mfma_ceiling(iters=2000):
    """Matrix-core rate of the ceiling kernel (one workgroup of four waves per
    compute unit, each wave 128 x 128 of v_mfma_f32_32x32x16_f16 on register
    operands): MFMAs alone, and with the GEMM's exact FP4 decode of the next
    operands interleaved; median of 3 runs of 10 back-to-back launches."""
    path = os.path.join(ROOT, "moe_nvfp4_quantize_amd", "libnvfp4_ceiling.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.ceiling_grid.restype = ctypes.c_uint32
    lib.ceiling_grid.argtypes = [ctypes.c_uint32]
    lib.ceiling_mfma.restype = ctypes.c_int
    lib.ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p]
    grid = lib.ceiling_grid(1)
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flops = grid * 4 * iters * 2 * 16 * (2 * 32 * 32 * 16)
    out = {}
    for label, dec in (("mfma_only", 0), ("mfma_with_decode", 1)):
        if lib.ceiling_mfma(sink.data_ptr(), iters, dec, stream()) != 0:
            return None
        ms = statistics.median([run_timed(lambda i: lib.ceiling_mfma(sink.data_ptr(), iters, dec, stream()), 10)
                                for _ in range(3)])
        tf = flops / (ms * 1e-3) / 1e12
        out[label] = dict(tflops=tf, frac_f16_peak=tf / F16_MFMA_PEAK_TFLOPS, ms=ms)
    out["note"] = ("f16 MFMA 32x32x16 with f32 accumulation, no memory or LDS traffic; the clock the chip "
                   "holds under this load sets it below the 2.5 PFLOP/s specification")
    return out


# ------------------------------------------------------------------- MoE


def moe_setup(B, name, static=False):
    cfg = W.WORKLOADS[name]
    inp = W.moe_inputs(name, device="cuda")
    wgu = B.nvfp4_quantize_batched(inp["w_gate_up"])
    wd = B.nvfp4_quantize_batched(inp["w_down"])
    del inp["w_gate_up"], inp["w_down"]
    torch.cuda.empty_cache()
    st = dict(cfg=cfg, name=name, k=inp["k"], static=static)
    nin = n_copies(tensor_bytes([inp["x"], inp["logits"]]))
    st["ins"] = [(inp["x"], inp["logits"])] + [(inp["x"].clone(), inp["logits"].clone()) for _ in range(nin - 1)]
    nw = n_copies(tensor_bytes(wgu) + tensor_bytes(wd))
    st["ws"] = [(wgu, wd)] + [(tuple(t.clone() for t in wgu), tuple(t.clone() for t in wd)) for _ in range(nw - 1)]
    if static:
        # calibrate the two activation scales (max over a batch of other tokens), untimed
        T_cal = min(cfg["T"], 2048)
        lg, xc = W.moe_calibration_inputs(name, T_cal, device="cuda")
        r = B.nvfp4_moe_route(lg, st["k"])
        xq = B.nvfp4_quantize(xc)
        h = B.nvfp4_moe_grouped_gemm(xq, r["src_row"], r["offsets"], T_cal * st["k"], wgu,
                                     epilogue=B.NVFP4_EPI_SILU_GATE, out_dtype=torch.float32)
        st["gx"] = xq[2].clone()
        st["gh"] = B.nvfp4_quantize(h)[2].clone()
        del h
    return st


def moe_step(B, st):
    T, k = st["cfg"]["T"], st["k"]
    R = T * k
    ins, ws = st["ins"], st["ws"]
    if st["static"]:
        names = ["route", "quantize_x", "gate_up", "down", "combine"]

        def step(i, tm=None):
            x, logits = ins[i % len(ins)]
            wgu, wd = ws[i % len(ws)]
            m = [tm.mark()] if tm else None
            r = B.nvfp4_moe_route(logits, k)
            if tm: m.append(tm.mark())
            xq = B.nvfp4_quantize(x, g=st["gx"])
            if tm: m.append(tm.mark())
            hq = B.nvfp4_moe_grouped_gemm_silu_nvfp4(xq, r["src_row"], r["offsets"], R, wgu, st["gh"])
            if tm: m.append(tm.mark())
            y = B.nvfp4_moe_grouped_gemm(hq, None, r["offsets"], R, wd, out_dtype=torch.bfloat16)
            if tm: m.append(tm.mark())
            B.nvfp4_moe_combine(y, r["topk_w"], r["inv"])
            if tm:
                m.append(tm.mark())
                for j, n in enumerate(names):
                    tm.add(n, m[j], m[j + 1])
        return step, names
    names = ["route", "quantize_x", "gate_up", "quantize_h", "down", "combine"]

    def step(i, tm=None):
        x, logits = ins[i % len(ins)]
        wgu, wd = ws[i % len(ws)]
        m = [tm.mark()] if tm else None
        r = B.nvfp4_moe_route(logits, k)
        if tm: m.append(tm.mark())
        xq = B.nvfp4_quantize(x)
        if tm: m.append(tm.mark())
        h = B.nvfp4_moe_grouped_gemm(xq, r["src_row"], r["offsets"], R, wgu,
                                     epilogue=B.NVFP4_EPI_SILU_GATE, out_dtype=torch.bfloat16)
        if tm: m.append(tm.mark())
        hq = B.nvfp4_quantize(h)
        if tm: m.append(tm.mark())
        y = B.nvfp4_moe_grouped_gemm(hq, None, r["offsets"], R, wd, out_dtype=torch.bfloat16)
        if tm: m.append(tm.mark())
        B.nvfp4_moe_combine(y, r["topk_w"], r["inv"])
        if tm:
            m.append(tm.mark())
            for j, n in enumerate(names):
                tm.add(n, m[j], m[j + 1])
    return step, names


def moe_report(st, step_ms, kstats, steps):
    cfg = st["cfg"]
    T, E, k, H, I = cfg["T"], cfg["E"], cfg["k"], cfg["H"], cfg["I"]
    R = T * k
    f_gu = 2.0 * R * 2 * I * H
    f_d = 2.0 * R * H * I
    flops = f_gu + f_d
    w_gu_b = 0.5625 * E * 2 * I * H
    w_d_b = 0.5625 * E * H * I
    gu_bytes = w_gu_b + 0.5625 * T * H + 2 * R * I  # weights, X packed once, h bf16
    d_bytes = w_d_b + 0.5625 * R * I + 2 * R * H    # weights, h packed, y bf16
    traffic = None if st["static"] else profiled_traffic(PROFILES[st["name"]], "moe_nvfp4_quantize_amd/csrc/gemm.hip")
    gu, dn = kstats["gate_up"], kstats["down"]
    kernel = "nvfp4 gemm_dma_kernel (grouped, SiLU gate" + (" -> NVFP4 h)" if st["static"] else ")")
    roof = roofline_entry(f_gu, gu_bytes, gu["mean_ms"], kernel, traffic)
    kern = {n: dict(s) for n, s in kstats.items()}
    kern["gate_up"].update(tflops=f_gu / (gu["mean_ms"] * 1e-3) / 1e12,
                           frac_f16_peak=f_gu / (gu["mean_ms"] * 1e-3) / 1e12 / F16_MFMA_PEAK_TFLOPS,
                           traffic=traffic, algorithmic_bytes=gu_bytes)
    kern["down"].update(tflops=f_d / (dn["mean_ms"] * 1e-3) / 1e12,
                        frac_f16_peak=f_d / (dn["mean_ms"] * 1e-3) / 1e12 / F16_MFMA_PEAK_TFLOPS,
                        traffic=None if st["static"] else profiled_traffic(
                            PROFILES[st["name"]], "moe_nvfp4_quantize_amd/csrc/gemm.hip", "down_traffic_bytes_per_launch"),
                        algorithmic_bytes=d_bytes)
    if "quantize_h" in kern:
        qh = quant_bytes(R * I, 2)
        kern["quantize_h"].update(gbs=qh / (kern["quantize_h"]["mean_ms"] * 1e-3) / 1e9, algorithmic_bytes=qh)
    return dict(ms_per_step=step_ms, value=flops / (step_ms * 1e-3) / 1e12, unit="TFLOP/s", steps=steps,
                roofline=roof, kernels=kern,
                config=dict(workload=st["name"], T=T, E=E, k=k, H=H, I=I, x="bf16", out="bf16",
                            experts="NVFP4 gate_up [2I x H] and down [H x I], quantized offline",
                            intermediates="h and y stored in bf16, combine in float32",
                            activation_scales="static (calibrated on 2048 other tokens), h quantized in the "
                                              "gate_up epilogue" if st["static"] else "dynamic",
                            rotation=dict(input_copies=len(st["ins"]), weight_copies=len(st["ws"]))))


def measure(B, name, steps, warmup, kernel_iters, static=False, dense_state=None):
    """Set up one workload, warm up, time `steps` steps as a whole and then
    `kernel_iters` steps with events around each kernel."""
    kind = W.WORKLOADS[name]["kind"]
    if kind == "linear":
        st = dense_state or dense_setup(B, name)
        step, names = dense_step(B, st)
    else:
        st = moe_setup(B, name, static=static)
        step, names = moe_step(B, st)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    step_ms = run_timed(step, steps)
    kstats = run_kernels(step, names, kernel_iters, first=steps)
    rep = dense_report(st, step_ms, kstats, steps) if kind == "linear" else moe_report(st, step_ms, kstats, steps)
    return st, rep


# ----------------------------------------------------------- CPU baseline


def cpu_host():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count() or 1
    # the GPU host's share is 16 cores whatever the machine has
    return model, nproc, max(1, min(16, nproc, int(os.environ.get("OMP_NUM_THREADS", nproc))))


def _limit_blas(n):
    from threadpoolctl import threadpool_limits
    return threadpool_limits(n)


def _pool_init():
    global _LIM
    _LIM = _limit_blas(1)


def _quantize_part(x, g):
    from oracle import nvfp4 as OQ
    OQ.quantize(x, g=g)
    return x.size


def _dequantize_part(q, s, g):
    from oracle import nvfp4 as OQ
    OQ.dequantize(q, s, g)
    return q.size * 2


class OracleRates:
    """Per-element and per-flop rates of the oracle's pieces on this host, on
    one core or on `threads` (row blocks over a process pool of that many
    workers for the element-wise pieces; BLAS threads for the products)."""

    def __init__(self, threads):
        self.threads = threads
        self.pool = None
        if threads > 1:
            import multiprocessing as mp
            from concurrent.futures import ProcessPoolExecutor
            self.pool = ProcessPoolExecutor(threads, mp_context=mp.get_context("forkserver"),
                                            initializer=_pool_init)
            list(self.pool.map(abs, range(threads)))  # start the workers before any timing

    def close(self):
        if self.pool is not None:
            self.pool.shutdown(wait=True)

    def _elementwise(self, fn, parts):
        t0 = time.perf_counter()
        if self.pool is None:
            with _limit_blas(1):
                n = sum(fn(*p) for p in parts)
        else:
            n = sum(self.pool.map(fn, *zip(*parts)))
        return (time.perf_counter() - t0) / n

    def quantize(self, x, g):
        """s per element of oracle.nvfp4.quantize (given g) on float32 rows x."""
        per = max(1, x.shape[0] // max(1, self.threads))
        return self._elementwise(_quantize_part, [(x[r:r + per], g) for r in range(0, x.shape[0], per)])

    def dequantize(self, t):
        q, s, g = t
        per = max(1, q.shape[0] // max(1, self.threads))
        return self._elementwise(_dequantize_part, [(q[r:r + per], s[r:r + per], g)
                                                    for r in range(0, q.shape[0], per)])

    def matmul(self, a, b):
        """s per flop of the float64 product a @ b.T (the oracle GEMM's product)."""
        with _limit_blas(self.threads):
            a @ b.T
            t0 = time.perf_counter()
            a @ b.T
            return (time.perf_counter() - t0) / (2.0 * a.shape[0] * b.shape[0] * a.shape[1])

    def amax(self, x):
        t0 = time.perf_counter()
        from oracle import nvfp4 as OQ
        OQ.global_scale(x)
        return time.perf_counter() - t0


def _median3(fn):
    vals = [fn() for _ in range(3)]
    return statistics.median(vals), vals


def cpu_dense(name, rates):
    """Oracle step time of a dense workload: global scale of X (whole X), the
    quantize of X (per element, on 256 rows), the GEMM's dequantize of both
    operands (per element, on 256 rows of each) and its float64 product (per
    flop, on a 256 x 1024 block), scaled to the full shapes."""
    import numpy as np
    from oracle import nvfp4 as OQ
    cfg = W.WORKLOADS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x, w = W.linear_inputs(name, device="cpu")
    xh = x.float().numpy()
    wh = w[:1024].float().numpy()
    gx, gw = OQ.global_scale(xh), OQ.global_scale(wh)
    xs = xh[:min(M, 256)]
    aq = OQ.quantize(xh[:min(M, 512)], g=gx)
    bq = OQ.quantize(wh, g=gw)
    A, Bm = OQ.dequantize(*aq), OQ.dequantize(*bq)
    a256 = (aq[0][:256], aq[1][:256], aq[2])
    b256 = (bq[0][:256], bq[1][:256], bq[2])

    def once():
        return (rates.amax(xh) + M * K * rates.quantize(xs, gx) + M * K * rates.dequantize(a256)
                + N * K * rates.dequantize(b256) + 2.0 * M * N * K * rates.matmul(A, Bm))
    step_s, runs = _median3(once)
    return step_s, runs, (f"global scale of all of X; quantize of {xs.shape[0]} rows; dequantize of 256 rows of "
                          f"each operand; float64 product {A.shape[0]}x{Bm.shape[0]}x{K}; scaled to "
                          f"{M}x{N}x{K}"), 2.0 * M * N * K


def cpu_moe(name, rates):
    """Oracle step time of an MoE workload: routing and permutation of all
    tokens (Python, one core), the quantize of X and of h (per element), the
    grouped GEMMs' dequantize of the gathered rows and of every expert's
    matrix (per element) and float64 products (per flop, measured on one
    expert's shapes), the SiLU gate (per element) and the combine (per token,
    on 512 tokens), scaled to the full layer."""
    import numpy as np
    from oracle import moe as OM
    from oracle import nvfp4 as OQ
    cfg = W.WORKLOADS[name]
    T, E, k, H, I = cfg["T"], cfg["E"], cfg["k"], cfg["H"], cfg["I"]
    R = T * k
    d = W.moe_inputs(name, device="cpu", weights=False)
    xh = d["x"].float().numpy()
    lh = d["logits"].numpy()
    gen = np.random.default_rng(5)
    wgu = (gen.standard_normal((2 * I, H)) * 0.02).astype(np.float32)
    wdn = (gen.standard_normal((H, I)) * 0.02).astype(np.float32)
    rows = max(1, R // E)
    xs = xh[:min(T, 256)]
    gx = OQ.global_scale(xh)
    aq = OQ.quantize(xh[:rows], g=gx)
    wq_gu, wq_d = OQ.quantize(wgu), OQ.quantize(wdn)
    hs = (gen.standard_normal((rows, I)) * 0.1).astype(np.float32)
    hq = OQ.quantize(hs)
    Agu, Wgu = OQ.dequantize(*aq), OQ.dequantize(*wq_gu)
    Ad, Wd = OQ.dequantize(*hq), OQ.dequantize(*wq_d)
    ysmp = gen.standard_normal((512 * k, H)).astype(np.float32)  # the routed rows of 512 tokens
    wts = np.abs(gen.standard_normal((512, k)))
    inv = gen.permutation(512 * k).reshape(512, k)

    def once():
        t0 = time.perf_counter()
        ids, _ = OM.route(lh, k)
        OM.permute(ids, E)
        t_route = time.perf_counter() - t0
        t0 = time.perf_counter()
        OM.silu_gate(np.zeros((rows, 2 * I)))
        t_silu = (time.perf_counter() - t0) / (rows * I)
        t0 = time.perf_counter()
        OM.combine(ysmp, wts, inv)
        t_comb = (time.perf_counter() - t0) / 512
        rq = rates.quantize(xs, gx)
        return (t_route + rates.amax(xh) + T * H * rq
                + R * H * rates.dequantize(aq) + E * 2 * I * H * rates.dequantize(wq_gu)
                + 2.0 * R * 2 * I * H * rates.matmul(Agu, Wgu) + R * I * t_silu
                + rates.amax(hs) * (R / rows) + R * I * rates.quantize(hs, OQ.global_scale(hs))
                + R * I * rates.dequantize(hq) + E * H * I * rates.dequantize(wq_d)
                + 2.0 * R * H * I * rates.matmul(Ad, Wd) + T * t_comb)
    step_s, runs = _median3(once)
    return step_s, runs, (f"routing + permutation of all {T} tokens; quantize of {xs.shape[0]} rows of X and "
                          f"{rows} rows of h; dequantize and float64 products at one expert's shapes ({rows} "
                          f"rows); SiLU gate and combine on samples; scaled to {E} experts, {R} routed rows"), \
        2.0 * R * 3 * I * H


def cpu_baselines(names):
    """{workload: cpu_baseline dict} for each name, one core and all cores."""
    model, nproc, threads = cpu_host()
    out = {}
    for label, n in (("one_core", 1), ("all_cores", threads)):
        rates = OracleRates(n)
        try:
            for name in names:
                fn = cpu_dense if W.WORKLOADS[name]["kind"] == "linear" else cpu_moe
                step_s, runs, sample, flops = fn(name, rates)
                out.setdefault(name, {})[label] = dict(step_s=step_s, runs_s=runs,
                                                       value=flops / step_s / 1e12, threads=n)
                out[name]["sample"] = sample
        finally:
            rates.close()
    res = {}
    for name, v in out.items():
        a = v["all_cores"]
        res[name] = dict(value=a["value"], unit="TFLOP/s", cores=a["threads"], kind="oracle",
                         sample=v["sample"] + " (3 repeats, median)", step_s=a["step_s"], runs_s=a["runs_s"],
                         one_core=dict(value=v["one_core"]["value"], step_s=v["one_core"]["step_s"],
                                       runs_s=v["one_core"]["runs_s"]),
                         cpu_model=model, host_cpus=nproc,
                         parallelism="element-wise oracle steps over a process pool of row blocks, float64 "
                                     "products on that many BLAS threads")
    return res


# ------------------------------------------------------------------- main


def library_reference(st, reps):
    """The platform libraries' GEMMs at the dense shape (context, not part of the path)."""
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
        ms = run_timed(lambda i: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16),
                       reps)
        out["fp8_scaled_mm"] = dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12)
        del a8, b8
    except Exception as ex:  # the library call is optional context
        out["fp8_scaled_mm"] = dict(error=str(ex)[:200])
    ab, bb = a.to(torch.bfloat16), b.to(torch.bfloat16)
    del a, b
    ms = run_timed(lambda i: ab @ bb.t(), reps)
    out["bf16_matmul"] = dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12)
    out["note"] = "platform GEMM libraries through torch at the same shape; context only"
    return out


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
    head = args.workload
    if args.configs == "all":
        others = [n for n in LARGE if n != head]
    elif args.configs == "none":
        others = []
    else:
        others = [n for n in args.configs.split(",") if n and n != head]
    iters = max(1, args.iters)

    # the other workloads first (each set up, measured and released in turn)
    configs = {}
    for name in others:
        print(f"bench: {name}", file=sys.stderr, flush=True)
        st, rep = measure(B, name, steps=iters, warmup=max(10, args.warmup), kernel_iters=iters)
        configs[name] = rep
        del st
        torch.cuda.empty_cache()

    # headline: W warm-up steps, exactly K timed steps, then the per-kernel pass
    kind = W.WORKLOADS[head]["kind"]
    print(f"bench: {head} (headline)", file=sys.stderr, flush=True)
    st, rep = measure(B, head, steps=args.steps, warmup=args.warmup, kernel_iters=max(args.steps, iters),
                      static=args.static_scales)
    extra = {}
    if kind == "linear":
        extra.update(quantizer_legs(B, st, iters))
        ceil = ceilings(st, iters)
        extra["ceilings"] = ceil
        extra["mfma_ceiling"] = mfma_ceiling()
        if ceil:
            for key in ("quantize_cold", "quantize_static_cold"):
                extra[key]["frac_read_write_ceiling"] = extra[key]["gbs"] / ceil["read_write"]["gbs"]
        if args.library_reference:
            extra["library_reference"] = library_reference(st, max(10, iters // 5))
    if args.copy_probe_mib:
        a = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
    del st
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: oracle baselines on the host", file=sys.stderr, flush=True)
        base = cpu_baselines([head] + others)
        cpu = base[head]
        for name in others:
            configs[name]["cpu_baseline"] = base[name]

    line = dict(metric=METRIC, value=rep["value"], unit=rep["unit"], n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=rep["ms_per_step"], higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="f16", data="synthetic", config=rep["config"],
                roofline=rep["roofline"], cpu_baseline=cpu, kernels=rep["kernels"], **extra,
                configs=configs,
                timing=(f"cold: inputs rotated over copies exceeding {ROTATE_BYTES >> 20} MB; the headline's "
                        f"{args.steps} steps between two events after {args.warmup} warm-up steps; per-kernel "
                        f"figures over {max(args.steps, iters)} launches (other workloads: {iters} steps, "
                        "then as many with per-kernel events); roofline from the mean kernel duration"))
    print(json.dumps(line))


if __name__ == "__main__":
    main()
