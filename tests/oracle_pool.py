"""The oracle over a process pool, for parity checks at full workload sizes.

Test infrastructure: the oracle itself is single-threaded NumPy; these helpers
only cut a check into row / column blocks, run the oracle on each block in a
worker process and bring back either its (small) packed results or the
statistics of a comparison done in the worker.  Workers are fresh interpreters
(forkserver) that import NumPy and the oracle only, never the GPU stack.

Element-wise bounds (GEMM outputs; see gemm_block_check):
  the GPU accumulates exact f16 products in float32, one MFMA (16 products)
  at a time: against the exact sum S = sum_k a_k b_k its error is at most
  (K/16 + 20) * 2^-24 * sum_k |a_k b_k| (each of the K/16 accumulations rounds
  once, the 16-product sums and the epilogue's scaling by a_g * b_g a few times
  more), and sum_k |a_k b_k| <= ||a|| ||b|| (Cauchy-Schwarz).  A bf16 output
  rounds that float32 value once more: one bf16 unit in the last place of the
  exact value (2^-7 relative to its binade) is added.
"""

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

U = 2.0 ** -24
_POOL = None


def n_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init_worker():
    global _LIMIT
    try:
        from threadpoolctl import threadpool_limits
        _LIMIT = threadpool_limits(1)  # one BLAS thread per worker: the pool is the parallelism
    except Exception:  # pragma: no cover
        _LIMIT = None


def pool():
    global _POOL
    if _POOL is None:
        _POOL = ProcessPoolExecutor(n_workers(), mp_context=mp.get_context("forkserver"),
                                    initializer=_init_worker)
    return _POOL


def shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True)
        _POOL = None


# ------------------------------------------------------------------ quantize


def _quantize_chunk(x, g):
    from oracle import nvfp4 as Q
    q, s, _ = Q.quantize(x, g=g)
    return q, s


def quantize_rows(x, g, rows_per_task=None):
    """The oracle's (q, s) of float32 x [rows, cols] under global scale g, by row blocks."""
    rows = x.shape[0]
    if rows_per_task is None:
        rows_per_task = max(1, min(rows, (4 << 20) // max(1, x.shape[1])))  # ~4 M elements per task
    futs = [pool().submit(_quantize_chunk, np.ascontiguousarray(x[r:r + rows_per_task]), g)
            for r in range(0, rows, rows_per_task)]
    parts = [f.result() for f in futs]
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _qdq_chunk(x, g, out):
    from oracle import qdq as D
    return D.qdq(x, g=g, out=out)[0]


def qdq_rows(x, g, out, rows_per_task=None):
    """The oracle's quantize-dequantize of float32 x [rows, cols] under global
    scale g ("f32" or "bf16" values), by row blocks."""
    rows = x.shape[0]
    if rows_per_task is None:
        rows_per_task = max(1, min(rows, (4 << 20) // max(1, x.shape[1])))
    futs = [pool().submit(_qdq_chunk, np.ascontiguousarray(x[r:r + rows_per_task]), g, out)
            for r in range(0, rows, rows_per_task)]
    return np.concatenate([f.result() for f in futs])


def _four6_chunk(x, g):
    from oracle import four_over_six as F
    q, s, _, took4 = F.quantize(x, g=g)
    return q, s, int(took4.sum())


def four_over_six_rows(x, g, rows_per_task=None):
    """The four-over-six oracle's (q, s) of float32 x [rows, cols] under global
    scale g, by row blocks, and how many blocks took the scale of 4."""
    rows = x.shape[0]
    if rows_per_task is None:
        rows_per_task = max(1, min(rows, (4 << 20) // max(1, x.shape[1])))
    futs = [pool().submit(_four6_chunk, np.ascontiguousarray(x[r:r + rows_per_task]), g)
            for r in range(0, rows, rows_per_task)]
    parts = [f.result() for f in futs]
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            sum(p[2] for p in parts))


# ---------------------------------------------------------------------- GEMM


def bf16_ulp(v):
    """Unit in the last place of bfloat16 at |v| (8 significant bits)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(a)) - 7).astype(np.int64))


def _stats(y, ref, err_bound, out_bf16):
    """Comparison of GPU output y with the oracle's float64 ref under an
    element-wise bound on the float32 result's error."""
    y = np.asarray(y, dtype=np.float64)
    bound = err_bound + (bf16_ulp(np.abs(ref) + err_bound) if out_bf16 else 4 * U * np.abs(ref))
    diff = np.abs(y - ref)
    if out_bf16:
        cmp = np.asarray(ref, dtype=np.float32)
        b = cmp.view(np.uint32).astype(np.uint64)  # round to bf16, nearest even
        cmp = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    else:
        cmp = ref
    ratio = diff / bound
    return dict(n=int(y.size), bad=int((diff > bound).sum()), max_ratio=float(ratio.max(initial=0.0)),
                finite=bool(np.isfinite(y).all()),
                num=float(((y - cmp) ** 2).sum()), den=float((cmp ** 2).sum()),
                num_raw=float(((y - ref) ** 2).sum()), den_raw=float((ref ** 2).sum()))


def merge(stats):
    out = dict(n=0, bad=0, max_ratio=0.0, finite=True, num=0.0, den=0.0, num_raw=0.0, den_raw=0.0)
    for s in stats:
        for k in ("n", "bad", "num", "den", "num_raw", "den_raw"):
            out[k] += s[k]
        out["max_ratio"] = max(out["max_ratio"], s["max_ratio"])
        out["finite"] &= s["finite"]
    out["rel_fro"] = (out["num"] / out["den"]) ** 0.5 if out["den"] > 0 else out["num"] ** 0.5
    out["rel_fro_raw"] = (out["num_raw"] / out["den_raw"]) ** 0.5 if out["den_raw"] > 0 else 0.0
    return out


def _row_norms(t):
    from oracle import nvfp4 as Q
    return np.sqrt((Q.dequantize(*t) ** 2).sum(axis=1))


def gemm_block_check(a, b, y, out_bf16):
    """Oracle GEMM of NVFP4 operands a = (q, s, g) [m, K], b = (q, s, g) [n, K]
    against the GPU's y [m, n]; returns _stats."""
    from oracle import gemm as OG
    ref = OG.gemm(*a, *b)
    K = a[0].shape[1] * 2
    err = (K / 16 + 20) * U * np.outer(_row_norms(a), _row_norms(b))
    return _stats(y, ref, err, out_bf16)


def silu_gate_block_check(a, b, h, out_bf16):
    """Gate_up GEMM with the SiLU gate: b is [2I, K] (gate rows first); the
    GPU's h [m, I].  Bound: the gate and up accumulation bounds carried
    through h = SiLU(gate) * up (|SiLU'| <= 1.1), plus (8 + 2 |gate|) float32
    units of h for the hardware base-2 exponential and reciprocal (the
    exponent's own rounding moves e^-z by about |z| units)."""
    from oracle import gemm as OG
    from oracle import moe as OM
    gu = OG.gemm(*a, *b)
    with np.errstate(over="ignore"):
        ref = OM.silu_gate(gu)
    K = a[0].shape[1] * 2
    I = gu.shape[1] // 2
    e = (K / 16 + 20) * U * np.outer(_row_norms(a), _row_norms(b))
    gate, up = gu[:, :I], gu[:, I:]
    with np.errstate(over="ignore"):
        sg = np.abs(gate / (1.0 + np.exp(-gate)))
    err = 1.1 * e[:, :I] * (np.abs(up) + e[:, I:]) + sg * e[:, I:] + (8 + 2 * np.abs(gate)) * U * np.abs(ref)
    return _stats(h, ref, err, out_bf16)


# ----------------------------------------------------------------------- FP8


def _fp8_encode_chunk(x, g):
    from oracle import fp8 as P
    return P.encode(x, g)


def fp8_encode_rows(x, g, rows_per_task=None):
    """The FP8 oracle's E4M3 codes of float32 x [rows, cols] under the
    per-tensor scale g, by row blocks."""
    rows = x.shape[0]
    if rows_per_task is None:
        rows_per_task = max(1, min(rows, (4 << 20) // max(1, x.shape[1])))
    futs = [pool().submit(_fp8_encode_chunk, np.ascontiguousarray(x[r:r + rows_per_task]), g)
            for r in range(0, rows, rows_per_task)]
    return np.concatenate([f.result() for f in futs])


def fp8_gemm_block_check(a, b, y, out_bf16):
    """Oracle FP8 GEMM of a = (q, g) [m, K] and b = (q, g) [n, K] (E4M3 codes,
    per-tensor scales) against the GPU's y [m, n]; returns _stats.  Bound: the
    products of two E4M3 values are exact in float32, but unlike the NVFP4
    products (few-bit values whose sums stay exact) their sums round.  However
    the matrix core orders the sum, each of its K additions rounded to float32
    errs by at most one unit in the last place of a partial sum bounded by
    sum_k |a_k b_k| (2 U relative, whatever the rounding mode), and the
    epilogue's scaling by a_g b_g adds a few roundings more: 2 (K + 20) U
    ||a|| ||b||."""
    from oracle import fp8 as P
    ref = P.gemm(*a, *b)
    K = a[0].shape[1]
    na = np.sqrt((P.dequantize(*a) ** 2).sum(axis=1))
    nb = np.sqrt((P.dequantize(*b) ** 2).sum(axis=1))
    return _stats(y, ref, 2 * (K + 20) * U * np.outer(na, nb), out_bf16)


def run(fn, tasks):
    """Submit fn(*task) for every task; results in task order."""
    futs = [pool().submit(fn, *t) for t in tasks]
    return [f.result() for f in futs]
