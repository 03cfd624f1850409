"""GPU parity of the FP8 (E4M3, per-tensor) W8A8 path against the oracle.

Quantized bytes and the scale must be bit-exact.  The GEMM bar is a relative
Frobenius error <= 1e-3 against the oracle's float64 product of the exactly
dequantized operands (bf16 outputs: against the oracle rounded to bf16).  GEMM
operands are the oracle's own bytes, uploaded; the full-size workload runs the
GPU quantizer too and the oracle quantizes the sampled rows itself (given its
own scales, computed from the whole tensors on the host).
"""

import numpy as np
import pytest
import torch

from oracle import fp8 as P
from oracle import gemm as G
from oracle.formats import e4m3_decode
from moe_nvfp4_quantize_amd import workloads as W

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def B():
    from moe_nvfp4_quantize_amd import nvfp4
    nvfp4.load_library()
    return nvfp4


def _host(t):
    return t.detach().float().cpu().numpy()


def _up(q, g):
    return (torch.from_numpy(np.ascontiguousarray(q)).cuda(),
            torch.tensor([float(g)], dtype=torch.float32, device="cuda"))


def _bf16_round(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _compare(y_gpu, y_ref, out_dtype, label):
    y = y_gpu.double().cpu().numpy()
    ref = _bf16_round(y_ref) if out_dtype == torch.bfloat16 else y_ref
    err = G.rel_fro_error(y, ref)
    print(f"[fp8 gemm] {label}: rel_fro={err:.3e}", flush=True)
    assert np.all(np.isfinite(y))
    assert err <= TOL, (label, err)
    return err


# ------------------------------------------------------------------ quantize


@pytest.mark.parametrize("rows,cols,dtype", [(16, 512, torch.float32), (300, 1040, torch.bfloat16),
                                             (1, 16, torch.float32), (2048, 2048, torch.bfloat16),
                                             (777, 4096, torch.float32)])
def test_quantize_dynamic_bit_exact(B, rows, cols, dtype):
    print(f"[fp8 quantize] dynamic {rows}x{cols} {dtype}", flush=True)
    x = W.random_matrix(rows, cols, seed=rows + cols, device="cuda", std=3.0)
    x = (x * torch.exp(W.random_matrix(1, cols, seed=7, device="cuda"))).to(dtype)
    q, g = B.nvfp4_fp8_quantize(x)
    torch.cuda.synchronize()
    rq, rg = P.quantize(_host(x))
    assert g.item() == rg
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_quantize_strided_rows_and_linear_16x512(B):
    x, w = W.linear_inputs("linear_16x512", device="cuda")
    big = torch.zeros((16, 640), device="cuda")
    big[:, :512] = x
    for t in (big[:, :512], w):
        q, g = B.nvfp4_fp8_quantize(t)
        rq, rg = P.quantize(_host(t))
        assert g.item() == rg
        np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_quantize_static_scale_saturates(B):
    x = W.random_matrix(64, 256, seed=3, device="cuda", std=20.0)
    g = torch.tensor([2.0 ** -3], dtype=torch.float32, device="cuda")  # 1/g = 8: |x| > 56 saturates
    q, gg = B.nvfp4_fp8_quantize(x, g=g)
    torch.cuda.synchronize()
    assert gg.item() == 2.0 ** -3
    rq, _ = P.quantize(_host(x), g=np.float32(2.0 ** -3))
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    assert ((rq & 0x7F) == 0x7E).any()


def test_quantize_zero_and_signed_zero(B):
    x = torch.zeros((8, 64), device="cuda")
    x[1, :] = -0.0
    q, g = B.nvfp4_fp8_quantize(x)
    assert g.item() == 1.0
    rq, _ = P.quantize(_host(x))
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    assert (q[1] == 0x80).all() and (q[0] == 0).all()


def test_quantize_representable_round_trip(B):
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 0x7F, (128, 256)).astype(np.uint8) | (rng.integers(0, 2, (128, 256)) << 7).astype(np.uint8)
    codes[0, 0] = 0x7E
    x = (e4m3_decode(codes) * 2.0 ** -7).astype(np.float32)
    q, g = B.nvfp4_fp8_quantize(torch.from_numpy(x).cuda())
    assert g.item() == 2.0 ** -7
    np.testing.assert_array_equal(P.dequantize(q.cpu().numpy(), g.item()), x.astype(np.float64))


def test_quantize_prefill_and_two_pass_sampled(B):
    """The 8192x5120 bf16 activation (single-read kernel) and an fp32 tensor
    too large for it (two-pass kernels): scale exact, sampled rows bit-exact."""
    x, _ = W.linear_inputs("prefill_8192x5120", device="cuda")
    big = W.random_matrix(4100, 5200, seed=5, device="cuda", std=2.0)
    for label, t in (("prefill 8192x5120 bf16", x), ("fp32 4100x5200 two-pass", big)):
        print(f"[fp8 quantize] {label}", flush=True)
        q, g = B.nvfp4_fp8_quantize(t)
        torch.cuda.synchronize()
        th = _host(t)
        rg = P.scale(th)
        assert g.item() == rg, label
        rows = np.array([0, 1, t.shape[0] - 1] + list(range(5, t.shape[0], 613)))
        rq = P.encode(th[rows], rg)
        np.testing.assert_array_equal(q[torch.as_tensor(rows, device="cuda")].cpu().numpy(), rq)
        del q


def test_quantize_back_to_back_calls(B):
    """The single-read kernel's cross-workgroup state carries over between calls."""
    for i, (r, c) in enumerate([(4096, 2048), (64, 128), (4096, 2048), (1000, 3008)]):
        x = W.random_matrix(r, c, seed=100 + i, device="cuda").to(torch.bfloat16)
        q, g = B.nvfp4_fp8_quantize(x)
        rq, rg = P.quantize(_host(x))
        assert g.item() == rg
        np.testing.assert_array_equal(q.cpu().numpy(), rq)


# ---------------------------------------------------------------------- GEMM


def test_one_hot_columns_bit_exact(B):
    """A one-hot A (1.0 at column k_i) returns column k_i of B times both
    scales: exposes any mismatch of K order between the operands, a transposed
    operand or a wrong row/column map in the epilogue."""
    rng = np.random.default_rng(2)
    for M, N, K in [(300, 260, 256), (40, 50, 1024), (33, 17, 80)]:
        b_q = rng.integers(0, 256, (N, K)).astype(np.uint8)
        b_q[(b_q & 0x7F) == 0x7F] = 0x38
        k_of = rng.integers(0, K, M)
        a_q = np.zeros((M, K), np.uint8)
        a_q[np.arange(M), k_of] = 0x38
        y = B.nvfp4_fp8_gemm(_up(a_q, 2.0), _up(b_q, 0.25), out_dtype=torch.float32)
        np.testing.assert_array_equal(y.double().cpu().numpy(), P.gemm(a_q, 2.0, b_q, 0.25))


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (100, 300, 512), (257, 513, 1024), (128, 256, 4096),
                                   (600, 200, 2048), (300, 200, 80), (64, 64, 16), (5, 1, 48), (1, 1, 128)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_ragged_shapes(B, M, N, K, out_dtype):
    rng = np.random.default_rng(M * 7 + N + K)
    x = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal(K))).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    a, b = P.quantize(x), P.quantize(w)
    y = B.nvfp4_fp8_gemm(_up(*a), _up(*b), out_dtype=out_dtype)
    _compare(y, P.gemm(*a, *b), out_dtype, f"{M}x{N}x{K}")


def _exact_fp8_operands(rng, rows, K):
    """Codes of 0, +-0.5, +-1, +-2: every partial sum of products is a small
    multiple of 1/4, exact in any float32 summation order."""
    return rng.choice(np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], dtype=np.uint8), size=(rows, K))


@pytest.mark.parametrize("M,N,K", [(64, 96, 256), (300, 260, 1024), (7, 33, 48)])
def test_exact_sums_are_bit_identical(B, M, N, K):
    rng = np.random.default_rng(M + N + K)
    a, b = _exact_fp8_operands(rng, M, K), _exact_fp8_operands(rng, N, K)
    y = B.nvfp4_fp8_gemm(_up(a, 0.5), _up(b, 4.0), out_dtype=torch.float32)
    np.testing.assert_array_equal(y.double().cpu().numpy(), P.gemm(a, 0.5, b, 4.0))


def test_output_row_stride(B):
    rng = np.random.default_rng(4)
    a = P.quantize(rng.standard_normal((20, 256)).astype(np.float32))
    b = P.quantize(rng.standard_normal((30, 256)).astype(np.float32))
    big = torch.full((20, 48), 7.0, device="cuda")
    B.nvfp4_fp8_gemm(_up(*a), _up(*b), out=big[:, :30])
    torch.cuda.synchronize()
    _compare(big[:, :30], P.gemm(*a, *b), torch.float32, "ldc 48")
    assert torch.all(big[:, 30:] == 7.0)


def test_prefill_8192x5120_sampled(B):
    """Full-size dense prefill linear in FP8 W8A8: GPU quantize of X and W, GEMM
    with bf16 output; sampled outputs against the oracle."""
    x, w = W.linear_inputs("prefill_8192x5120", device="cuda")
    print("[fp8 gemm] prefill 8192x25600x5120: quantize + GEMM on the GPU", flush=True)
    qa, qb = B.nvfp4_fp8_quantize(x), B.nvfp4_fp8_quantize(w)
    y = B.nvfp4_fp8_gemm(qa, qb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xh, wh = _host(x), _host(w)
    ga, gb = P.scale(xh), P.scale(wh)
    assert qa[1].item() == ga and qb[1].item() == gb
    rows = np.array([0, 1, 255, 256, 8191] + list(range(3, 8192, 257)))
    cols = np.array([0, 1, 255, 256, 25599] + list(range(11, 25600, 401)))
    ref = P.gemm(P.encode(xh[rows], ga), ga, P.encode(wh[cols], gb), gb)
    ys = y[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")]
    _compare(ys, ref, torch.bfloat16, "prefill sampled")
    assert torch.isfinite(y.float()).all()


def test_deterministic(B):
    x, w = W.linear_inputs("prefill_8192x5120", device="cuda", M=512)
    qa, qb = B.nvfp4_fp8_quantize(x), B.nvfp4_fp8_quantize(w[:2048].contiguous())
    y1 = B.nvfp4_fp8_gemm(qa, qb)
    y2 = B.nvfp4_fp8_gemm(qa, qb)
    assert torch.equal(y1, y2)
