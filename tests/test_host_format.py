"""The kernels' format helpers (csrc/nvfp4_format.hpp), built for the host with
hipcc, against the oracle.  No GPU: this checks the encode logic the quantize
kernel uses before any kernel runs.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import nvfp4 as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_nvfp4_quantize_amd", "csrc")


@pytest.fixture(scope="module")
def helper(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("fmt") / "format_check")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                    "-ffp-contract=off", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "host", "format_check.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(lines):
        r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                           check=True)
        return r.stdout.split("\n")[:-1]
    return run


def _bits(a):
    return [f"{int(b):08x}" for b in np.asarray(a, dtype=np.float32).view(np.uint32)]


def _neigh(vals, n=4):
    out = []
    for v in vals:
        v = np.float32(v)
        up = dn = v
        out.append(v)
        for _ in range(n):
            up = np.nextafter(up, np.float32(np.inf), dtype=np.float32)
            dn = np.nextafter(dn, np.float32(-np.inf), dtype=np.float32)
            out += [up, dn]
    return np.array(out, dtype=np.float32)


def test_e2m1_encode_matches_oracle(helper):
    rng = np.random.default_rng(1)
    grid = list(F.E2M1_MAGNITUDES) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 1e30]
    pts = np.concatenate([_neigh(grid + [-g for g in grid]),
                          rng.uniform(-7, 7, 100000).astype(np.float32),
                          np.array([0.0, -0.0, 1e-40, -1e-40], dtype=np.float32)])
    got = np.array([int(v) for v in helper([f"e2m1 {b}" for b in _bits(pts)])])
    np.testing.assert_array_equal(got, F.e2m1_encode(pts))


def test_e4m3_encode_and_value_match_oracle(helper):
    rng = np.random.default_rng(2)
    mids = (F.E4M3_NONNEG[1:] + F.E4M3_NONNEG[:-1]) / 2
    pts = np.concatenate([_neigh(list(F.E4M3_NONNEG) + list(mids)),
                          np.exp(rng.uniform(np.log(1e-7), np.log(448), 50000)).astype(np.float32)])
    pts = pts[(pts >= 0) & (pts <= 448)]
    got = np.array([int(v) for v in helper([f"e4m3 {b}" for b in _bits(pts)])])
    np.testing.assert_array_equal(got, F.e4m3_encode(pts))
    vals = helper([f"e4m3v {c}" for c in range(1, 127)])
    got_v = np.array([int(v, 16) for v in vals], dtype=np.uint32).view(np.float32)
    np.testing.assert_array_equal(got_v.astype(np.float64), F.e4m3_decode(np.arange(1, 127)))


def test_block_scale_step_matches_oracle(helper):
    """The kernel's per-block step (scale code and reciprocal) on many (bmax, g)."""
    rng = np.random.default_rng(3)
    g = (np.exp(rng.uniform(np.log(1e-8), np.log(10.0), 3000)) / 2688).astype(np.float32)
    frac = np.exp(rng.uniform(np.log(1e-7), 0.0, 3000))
    bmax = (g.astype(np.float64) * 2688 * frac).astype(np.float32)
    bmax[:50] = 0.0
    bmax[50:100] = (g[50:100].astype(np.float64) * 2688).astype(np.float32)
    lines = [f"scale {a} {b}" for a, b in zip(_bits(bmax), _bits(g))]
    out = [l.split() for l in helper(lines)]
    codes = np.array([int(c) for c, _ in out], dtype=np.uint8)
    recips = np.array([int(r, 16) for _, r in out], dtype=np.uint32).view(np.float32)
    for i in range(len(g)):
        x = np.zeros((1, 16), dtype=np.float32)
        x[0, 0] = bmax[i]
        s = Q.block_scales(x, g[i])[0, 0]
        assert codes[i] == s, (bmax[i], g[i])
        sv = np.float32(F.e4m3_decode(s))
        assert recips[i] == np.float32(1.0) / np.float32(sv * g[i])


def test_bf16_rounding_matches_torch(helper):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.00390625, 1.01171875]  # exact ties
    got = np.array([int(v, 16) for v in helper([f"bf16 {b}" for b in _bits(x)])], dtype=np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_fast_division(helper):
    rng = np.random.default_rng(5)
    ds = [1, 2, 3, 7, 16, 32, 320, 321, 4096, 65535, 151936 // 16, 2 ** 31 - 1]
    cases = [(int(n), d) for d in ds for n in list(rng.integers(0, 2 ** 31, 200)) + [0, d - 1, d, 2 ** 31 - 1]]
    got = helper([f"div {n} {d}" for n, d in cases])
    assert [int(v) for v in got] == [n // d for n, d in cases]


def _topk_host(helper, rows, k):
    lines = [f"topk {r.shape[0]} {k} " + " ".join(_bits(r)) for r in rows]
    return np.array([[int(v) for v in l.split()] for l in helper(lines)], dtype=np.int64)


def test_topk_selection_matches_oracle_on_finite_rows(helper):
    """The top-k kernel's ranking, run on the host, against the oracle's sort:
    larger logit first, ties to the lower expert id (rows with many ties)."""
    from oracle import moe as OM
    rng = np.random.default_rng(6)
    rows = rng.standard_normal((200, 40)).astype(np.float32)
    rows[:50] = np.round(rows[:50])  # heavy ties
    rows[50:60] = 0.0
    rows[60, 5] = -0.0
    rows[61] = -np.inf
    rows[62, :7] = np.inf
    ids, _ = OM.topk(np.where(np.isinf(rows), np.sign(rows) * 1e38, rows).astype(np.float32), 9)
    got = _topk_host(helper, rows, 9)
    np.testing.assert_array_equal(got[:61], ids[:61])
    assert list(got[61]) == list(range(9))          # all -inf: lowest ids
    assert list(got[62][:7]) == list(range(7))       # the seven +inf first


def test_topk_selection_never_runs_out_on_nan_rows(helper):
    """A NaN logit ranks as -infinity: a row with fewer than k non-NaN logits,
    an all-NaN row included, still gets k distinct experts in [0, E), the
    finite logits first in their order, then the NaN ones by lower id."""
    rng = np.random.default_rng(7)
    E, k = 64, 10
    rows = rng.standard_normal((6, E)).astype(np.float32)
    rows[0] = np.nan                                  # all NaN
    rows[1, 3:] = np.nan                              # 3 finite logits, k = 10
    rows[2, ::2] = np.nan                             # half NaN
    rows[3, :] = np.nan
    rows[3, 40] = -np.inf                             # -inf ties with NaN: lower id first
    rows[4, 10:20] = np.nan                           # NaNs only among low ranks
    got = _topk_host(helper, rows, k)
    for r, ids in zip(rows, got):
        assert len(set(ids)) == k and ids.min() >= 0 and ids.max() < E
        fin = np.flatnonzero(~np.isnan(r) & ~np.isneginf(r))
        nfin = min(k, fin.size)
        order = sorted(fin, key=lambda e: (-r[e], e))[:nfin]
        assert list(ids[:nfin]) == order
    assert list(got[0]) == list(range(k))
    assert list(got[1][3:]) == list(range(3, 10))
    assert list(got[3]) == list(range(k))
