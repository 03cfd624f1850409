"""GPU parity of nvfp4_gemm against the oracle (float64 product of exactly
dequantized operands).

Bar: relative Frobenius error <= 1e-3.  For bf16 outputs the oracle is rounded
to bf16 (round to nearest even) before comparing, since bf16's 8 significant
bits alone give about 2e-3.  Crafted operands whose float32 sums are exact must
come out bit-identical.

Operands fed to the GPU are the oracle's own quantized bytes, uploaded; the
full-size workloads instead run the GPU quantizer too and the oracle quantizes
the sampled rows of both operands itself (given its own global scales).
"""

import numpy as np
import pytest
import torch

from oracle import gemm as G
from oracle import nvfp4 as Q
from oracle.formats import e2m1_decode
from moe_nvfp4_quantize_amd import workloads as W

import oracle_pool as OP

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def B():
    from moe_nvfp4_quantize_amd import nvfp4
    nvfp4.load_library()
    return nvfp4


def _up(t):
    q, s, g = t
    return (torch.from_numpy(np.ascontiguousarray(q)).cuda(), torch.from_numpy(np.ascontiguousarray(s)).cuda(),
            torch.tensor([float(g)], dtype=torch.float32, device="cuda"))


def _bf16_round(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _host(t):
    return t.detach().float().cpu().numpy()


def _compare(y_gpu, y_ref, out_dtype, label, operands=None):
    """Relative Frobenius error against the oracle (bf16-rounded for bf16
    outputs) within TOL; with the operands (a, b) also every element within the
    float32 accumulation bound (K/16 + 20) 2^-24 |a_m| |b_n| (plus one bf16
    unit of the exact value for bf16 outputs, tests/oracle_pool.py)."""
    y = y_gpu.double().cpu().numpy()
    raw = G.rel_fro_error(y, y_ref)
    if out_dtype == torch.bfloat16:
        err = G.rel_fro_error(y, _bf16_round(y_ref))
    else:
        err = raw
    extra = ""
    if operands is not None:
        a, b = operands
        K = a[0].shape[1] * 2
        bound = (K / 16 + 20) * OP.U * np.outer(OP._row_norms(a), OP._row_norms(b))
        st = OP._stats(y, y_ref, bound, out_dtype == torch.bfloat16)
        extra = f", element-wise: {st['bad']} of {st['n']} past the bound (max ratio {st['max_ratio']:.3f})"
    print(f"[gemm] {label}: rel_fro={err:.3e} (vs raw fp64 {raw:.3e}){extra}", flush=True)
    assert np.all(np.isfinite(y))
    assert err <= TOL, (label, err)
    if operands is not None:
        assert st["bad"] == 0, (label, st["bad"], st["max_ratio"])
    return err


def _run(B, a, b, out_dtype):
    return B.nvfp4_gemm(_up(a), _up(b), out_dtype=out_dtype)


def test_linear_16x512(B):
    x, w = W.linear_inputs("linear_16x512")
    a, b = Q.quantize(x.numpy()), Q.quantize(w.numpy())
    y = _run(B, a, b, torch.float32)
    err = _compare(y, G.gemm(*a, *b), torch.float32, "linear_16x512")
    assert err < 1e-6  # float32 accumulation of exact products


def test_linear_16x512_through_gpu_quantizer(B):
    x, w = W.linear_inputs("linear_16x512", device="cuda")
    qa, qb = B.nvfp4_quantize(x), B.nvfp4_quantize(w)
    y = B.nvfp4_gemm(qa, qb, out_dtype=torch.float32)
    ref = G.gemm(*Q.quantize(_host(x)), *Q.quantize(_host(w)))
    assert _compare(y, ref, torch.float32, "linear_16x512 end to end") < 1e-6


def _exact_operands(rng, rows, K):
    """Codes in {0, +-0.5, +-1, +-2}, scales powers of two in [2^-3, 2^3], g = 1."""
    codes = rng.choice(np.array([0, 1, 2, 4, 9, 10, 12], dtype=np.uint8), size=(rows, K))
    s = rng.choice(np.array([0x20, 0x28, 0x30, 0x38, 0x40, 0x48, 0x50], dtype=np.uint8), size=(rows, K // 16))
    return Q.pack_codes(codes), s, np.float32(1.0)


@pytest.mark.parametrize("M,N,K", [(64, 96, 256), (130, 70, 512), (7, 33, 48), (128, 76800, 256)])
def test_exact_sums_are_bit_identical(B, M, N, K):
    rng = np.random.default_rng(M + N + K)
    a, b = _exact_operands(rng, M, K), _exact_operands(rng, N, K)
    y = _run(B, a, b, torch.float32).double().cpu().numpy()
    np.testing.assert_array_equal(y, G.gemm(*a, *b))


def test_every_code_and_scale_decodes_exactly(B):
    """A row per (scale, code pair): B picks single elements, so C holds A's decoded values."""
    K = 32
    scales = np.arange(1, 127, dtype=np.uint8)
    rows = []
    for sc in scales:
        codes = np.zeros(K, dtype=np.uint8)
        codes[:16] = np.arange(16)
        codes[16:] = np.arange(15, -1, -1)
        rows.append(codes)
    codes = np.stack(rows)
    a = (Q.pack_codes(codes), np.stack([np.array([sc, sc], dtype=np.uint8) for sc in scales]), np.float32(2.0))
    # B: one-hot rows, code 2 (= 1.0) at column n, scale 1.0 (0x38)
    bc = np.zeros((K, K), dtype=np.uint8)
    bc[np.arange(K), np.arange(K)] = 2
    b = (Q.pack_codes(bc), np.full((K, K // 16), 0x38, dtype=np.uint8), np.float32(0.5))
    y = _run(B, a, b, torch.float32).double().cpu().numpy()
    np.testing.assert_array_equal(y, Q.dequantize(*a) * 0.5)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (37, 200, 272), (130, 129, 512), (5, 300, 48),
                                   (256, 256, 768), (129, 1, 4096), (100, 300, 512), (1, 513, 256)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_ragged_shapes(B, M, N, K, out_dtype):
    rng = np.random.default_rng(M * N + K)
    x = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal(K))).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    a, b = Q.quantize(x), Q.quantize(w)
    y = _run(B, a, b, out_dtype)
    _compare(y, G.gemm(*a, *b), out_dtype, f"ragged {M}x{N}x{K}", operands=(a, b))


def _up_at(t, q_off, s_off):
    """Upload (q, s, g) with q and s starting q_off and s_off bytes past a
    16-byte boundary (dense rows)."""
    q, s, g = t

    def place(a, off):
        flat = torch.empty(a.size + 32, dtype=torch.uint8, device="cuda")
        base = (-flat.data_ptr()) % 16 + off
        v = flat[base:base + a.size].view(a.shape)
        v.copy_(torch.from_numpy(np.ascontiguousarray(a)))
        assert v.data_ptr() % 16 == off
        return v
    return place(q, q_off), place(s, s_off), torch.tensor([float(g)], dtype=torch.float32, device="cuda")


# Operands off the 16-byte (codes) or 8-byte (scales) alignment the direct-to-
# LDS kernel needs: accepted, and computed by the general kernel.
@pytest.mark.parametrize("which", ["a codes", "b scales", "all"])
@pytest.mark.parametrize("M,N,K", [(130, 300, 512), (64, 256, 1024)])
def test_misaligned_operands(B, which, M, N, K):
    rng = np.random.default_rng(M + N + K + len(which))
    a = _random_nvfp4(rng, M, K, 2.0 ** -6)
    b = _random_nvfp4(rng, N, K, 2.0 ** -7)
    offs = {"a codes": ((1, 0), (0, 0)), "b scales": ((0, 0), (0, 3)), "all": ((5, 1), (9, 2))}[which]
    y = B.nvfp4_gemm(_up_at(a, *offs[0]), _up_at(b, *offs[1]), out_dtype=torch.float32)
    _compare(y, G.gemm(*a, *b), torch.float32, f"misaligned {which} {M}x{N}x{K}", operands=(a, b))


def _random_nvfp4(rng, rows, K, g):
    """Operands straight in the format: any code byte, block scales from 0.25
    to 15 (E4M3 codes 0x28 .. 0x57)."""
    return (rng.integers(0, 256, (rows, K // 2), dtype=np.uint8),
            rng.integers(0x28, 0x58, (rows, K // 16), dtype=np.uint8), np.float32(g))


# Tile walks on a 256-CU device (tiles of 128 rows for M <= 128, else 256; 256
# columns): a last round at most half full runs each of its tiles as two
# halves of rows, and a product of at most 128 tiles runs every tile that way.
@pytest.mark.parametrize("M,N,K,out_dtype", [
    (1000, 17000, 1024, torch.float32),   # 268 tiles: 12 split, ragged last rows 768..999
    (100, 90000, 1024, torch.bfloat16),   # 352 tiles of 128 rows: 96 split, halves of 64 and 36 rows
    (100, 3000, 1024, torch.float32),     # 12 tiles, all split
    (65, 1000, 1024, torch.float32),      # second halves hold one row
    (129, 700, 256, torch.bfloat16),      # 256-row tiles, K with no persistent walk
    (300, 5000, 2048, torch.float32),     # 40 tiles in two tile rows, all split
    (250, 36000, 1024, torch.float32),    # 141 tiles: one each, none split
])
def test_split_tile_walks_full_output(B, M, N, K, out_dtype):
    rng = np.random.default_rng(M + N + K)
    a, b = _random_nvfp4(rng, M, K, 2.0 ** -4), _random_nvfp4(rng, N, K, 2.0 ** -6)
    y = _run(B, a, b, out_dtype)
    _compare(y, G.gemm(*a, *b), out_dtype, f"walk {M}x{N}x{K}", operands=(a, b))


# Seeded random shapes (K from 256 to 3072, M up to 700, N up to 40000) plus
# persistent walks with whole rounds (K % 1024 == 0, more tiles than compute
# units, with and without a split last round); full outputs against the oracle.
@pytest.mark.parametrize("M,N,K", [(82, 14634, 256), (62, 7258, 1024), (26, 32132, 768), (344, 16484, 2048),
                                   (92, 22309, 768), (423, 9234, 256), (154, 23826, 2048), (221, 38386, 1024),
                                   (248, 33185, 1280), (123, 37718, 1280),
                                   (700, 30000, 1024), (128, 80000, 1024), (513, 20000, 2048)])
def test_random_shapes_full_output(B, M, N, K):
    rng = np.random.default_rng(M * 131 + N + K)
    a, b = _random_nvfp4(rng, M, K, 2.0 ** -5), _random_nvfp4(rng, N, K, 2.0 ** -7)
    out_dtype = torch.bfloat16 if (M + N) % 2 else torch.float32
    y = _run(B, a, b, out_dtype)
    _compare(y, G.gemm(*a, *b), out_dtype, f"random {M}x{N}x{K}", operands=(a, b))


# Products of at most 128 rows whose 256-column tiles would leave a partly
# filled last round run on 320-column tiles (2 x 2 waves of 64 x 160) when that
# takes fewer rounds of a 256-CU device: one launch per tile (K % 1024 != 0) or
# a persistent walk, ragged N, 33..64 rows (one 32-row group per wave row).
@pytest.mark.parametrize("M,N,K", [(128, 76800, 256), (100, 70001, 512), (37, 76837, 1024), (65, 160000, 2048)])
def test_wide_skinny_tiles_full_output(B, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    a, b = _random_nvfp4(rng, M, K, 2.0 ** -5), _random_nvfp4(rng, N, K, 2.0 ** -7)
    for out_dtype in (torch.bfloat16, torch.float32):
        y = _run(B, a, b, out_dtype)
        _compare(y, G.gemm(*a, *b), out_dtype, f"320-column tiles {M}x{N}x{K}", operands=(a, b))


def test_output_row_stride(B):
    rng = np.random.default_rng(1)
    a = Q.quantize(rng.standard_normal((20, 64)).astype(np.float32))
    b = Q.quantize(rng.standard_normal((30, 64)).astype(np.float32))
    big = torch.full((20, 48), 7.0, device="cuda")
    B.nvfp4_gemm(_up(a), _up(b), out=big[:, :30])
    torch.cuda.synchronize()
    _compare(big[:, :30], G.gemm(*a, *b), torch.float32, "ldc 48", operands=(a, b))
    assert torch.all(big[:, 30:] == 7.0)


def _sampled_workload(B, name, rows, cols, out_dtype=torch.bfloat16):
    x, w = W.linear_inputs(name, device="cuda")
    print(f"[gemm] {name}: quantize + GEMM on the GPU", flush=True)
    qa, qb = B.nvfp4_quantize(x), B.nvfp4_quantize(w)
    y = B.nvfp4_gemm(qa, qb, out_dtype=out_dtype)
    torch.cuda.synchronize()
    xh, wh = _host(x), _host(w)
    ga, gb = Q.global_scale(xh), Q.global_scale(wh)
    assert qa[2].item() == ga and qb[2].item() == gb
    ra = Q.quantize(xh[rows], g=ga)
    rb = Q.quantize(wh[cols], g=gb)
    ref = G.gemm(*ra, *rb)
    ys = y[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")]
    _compare(ys, ref, out_dtype, f"{name} sampled {len(rows)}x{len(cols)}")
    yh = y.float()
    assert torch.isfinite(yh).all()


def test_prefill_8192x5120_sampled(B):
    rows = np.array([0, 1, 127, 128, 4095, 8191] + list(range(3, 8192, 257)))
    cols = np.array([0, 1, 255, 256, 25599] + list(range(11, 25600, 401)))
    _sampled_workload(B, "prefill_8192x5120", rows, cols)


def test_lmhead_128x151936_sampled(B):
    rows = np.arange(128)
    cols = np.array([0, 1, 151935, 151808, 151807] + list(range(5, 151936, 1499)))
    _sampled_workload(B, "lmhead_128x151936", rows, cols)


def test_deterministic(B):
    x, w = W.linear_inputs("prefill_8192x5120", device="cuda", M=256)
    w = w[:1024].contiguous()
    qa, qb = B.nvfp4_quantize(x), B.nvfp4_quantize(w)
    y1 = B.nvfp4_gemm(qa, qb)
    y2 = B.nvfp4_gemm(qa, qb)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("g_exp", [-4, -130])
def test_bf16_output_is_rounded_f32_output(B, g_exp):
    """The bf16 epilogue stores the float32 result rounded to nearest even,
    bit for bit, subnormal results included (tiny global scales): the same
    operands through the float32 and the bf16 output paths."""
    rng = np.random.default_rng(17 - g_exp)
    a = _random_nvfp4(rng, 300, 1024, 2.0 ** g_exp)
    b = _random_nvfp4(rng, 520, 1024, 2.0 ** -6)
    y32 = _run(B, a, b, torch.float32)
    y16 = _run(B, a, b, torch.bfloat16)
    torch.cuda.synchronize()
    want = y32.cpu().to(torch.bfloat16)
    assert torch.equal(y16.cpu().view(torch.int16), want.view(torch.int16))
    if g_exp < -126:
        assert (y32.abs() < 2.0 ** -126).float().mean().item() > 0.05  # many subnormal results
