"""GPU parity of nvfp4_quantize / nvfp4_quantize_batched against the oracle.

Bar: q, s and g bit-exact.  Full tensors where the oracle finishes in seconds;
at the full workload sizes, the global scale is checked in full and the codes
and scales of sampled rows (the oracle quantizes any row given g).
"""

import numpy as np
import pytest
import torch

from oracle import nvfp4 as Q
from moe_nvfp4_quantize_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from moe_nvfp4_quantize_amd import nvfp4
    nvfp4.load_library()
    return nvfp4


def _host(t):
    return t.detach().float().cpu().numpy()


def _check_full(B, x, g_static=None):
    print(f"[quantize] shape={tuple(x.shape)} dtype={x.dtype} static={g_static is not None}", flush=True)
    g_in = None if g_static is None else torch.tensor([g_static], dtype=torch.float32, device=x.device)
    q, s, g = B.nvfp4_quantize(x, g=g_in)
    torch.cuda.synchronize()
    rq, rs, rg = Q.quantize(_host(x), g=g_static)
    assert g.item() == rg
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_linear_16x512_x_and_w(B):
    x, w = W.linear_inputs("linear_16x512", device="cuda")
    _check_full(B, x)
    _check_full(B, w)


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (7, 4096 + 16), (129, 272), (1000, 32)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged_shapes(B, rows, cols, dtype):
    x = W.random_matrix(rows, cols, seed=rows * 7 + cols, dtype=dtype, device="cuda", std=3.0)
    _check_full(B, x)


def test_strided_rows_take_the_unaligned_path(B):
    base = W.random_matrix(33, 96 + 3, seed=4, dtype=torch.bfloat16, device="cuda")
    x = base[:, :96]  # row stride 99 elements: not 16-byte aligned
    q, s, g = B.nvfp4_quantize(x)
    rq, rs, rg = Q.quantize(_host(x))
    assert g.item() == rg
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("rows,cols,dtype", [(300, 1024, torch.bfloat16), (100, 512, torch.float32),
                                             (8200, 6144, torch.bfloat16)])
def test_misaligned_base_takes_the_unaligned_path(B, rows, cols, dtype):
    """Dense rows starting one element past a 16-byte boundary: accepted and
    quantized by the unaligned path (single-read for the first two shapes,
    two-pass for the last), bit-exact."""
    flat = W.random_matrix(1, rows * cols + 8, seed=rows + cols, dtype=dtype, device="cuda").view(-1)
    x = flat[1:1 + rows * cols].view(rows, cols)
    assert x.data_ptr() % 16 != 0
    if rows * cols > 10_000_000:
        _sampled(B, x, torch.tensor([0, 1, rows // 2, rows - 1] + list(range(7, rows, 997)), device="cuda"))
    else:
        _check_full(B, x)


def test_degenerate_values(B):
    z = torch.zeros((4, 64), device="cuda")
    _check_full(B, z)
    _check_full(B, -z)  # negative zero keeps its sign bit: codes 0x8
    one_hot = torch.zeros((2, 48), device="cuda")
    one_hot[1, 20] = -3.0
    _check_full(B, one_hot)
    tiny = W.random_matrix(8, 64, seed=5, device="cuda") * 1e-25
    _check_full(B, tiny)
    huge = W.random_matrix(8, 64, seed=6, device="cuda") * 1e30
    _check_full(B, huge)
    # exact E2M1 midpoints after scaling: amax 2688 -> g = 1, block scale 448
    mids = torch.tensor([[2688.0] + [448.0 * m for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] * 2
                         + [0.0] * 1], device="cuda")
    _check_full(B, mids[:, :16])


def test_representable_round_trip(B):
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(64, 256)).astype(np.uint8)
    codes[:, ::16] = 7
    s = rng.integers(1, 127, size=(64, 16)).astype(np.uint8)
    s[0, 0] = 0x7E
    from oracle.formats import e2m1_decode, e4m3_decode
    x = (e2m1_decode(codes).reshape(64, 16, 16) * e4m3_decode(s)[..., None]).reshape(64, 256) * 2.0 ** -6
    xt = torch.from_numpy(x.astype(np.float32)).cuda()
    q, sg, g = B.nvfp4_quantize(xt)
    assert g.item() == 2.0 ** -6
    np.testing.assert_array_equal(sg.cpu().numpy(), s)
    np.testing.assert_array_equal(q.cpu().numpy(), Q.pack_codes(codes))


def test_static_global_scale(B):
    x, _ = W.linear_inputs("linear_16x512", device="cuda")
    g = Q.global_scale(_host(x))
    _check_full(B, x, g_static=float(g))
    _check_full(B, x, g_static=float(np.float32(g) / np.float32(64)))  # saturating
    _check_full(B, x, g_static=float(np.float32(g) * np.float32(1000)))  # tiny scales


def test_empty_tensor_dynamic_gives_unit_global(B):
    x = torch.zeros((0, 64), device="cuda")
    q, s, g = B.nvfp4_quantize(x)
    assert g.item() == 1.0 and q.numel() == 0


def _sampled(B, x, rows):
    q, s, g = B.nvfp4_quantize(x)
    torch.cuda.synchronize()
    rg = Q.global_scale(_host(x))
    assert g.item() == rg
    xs = _host(x[rows])
    rq, rs, _ = Q.quantize(xs, g=rg)
    np.testing.assert_array_equal(s[rows].cpu().numpy(), rs)
    np.testing.assert_array_equal(q[rows].cpu().numpy(), rq)
    # properties over the whole tensor: scales positive finite, max 448 exactly
    sh = s.cpu().numpy()
    assert sh.max() == 0x7E and sh.min() >= 1 and np.all((sh & 0x7F) != 0x7F)
    return q, s, g


def test_prefill_8192x5120_activation_sampled(B):
    x, _ = W.linear_inputs("prefill_8192x5120", device="cuda")
    print("[quantize] prefill X 8192x5120 bf16", flush=True)
    rows = torch.tensor([0, 1, 2, 777, 4095, 4096, 8190, 8191] + list(range(100, 8192, 331)), device="cuda")
    _sampled(B, x, rows)


def test_prefill_8192x5120_weight_sampled(B):
    _, w = W.linear_inputs("prefill_8192x5120", device="cuda", M=1)
    print("[quantize] prefill W 25600x5120 bf16", flush=True)
    rows = torch.tensor([0, 1, 12799, 12800, 25599] + list(range(7, 25600, 997)), device="cuda")
    _sampled(B, w, rows)


def test_lmhead_weight_sampled(B):
    _, w = W.linear_inputs("lmhead_128x151936", device="cuda", M=1)
    print("[quantize] lm_head W 151936x2048 bf16", flush=True)
    rows = torch.tensor([0, 151935] + list(range(3, 151936, 4999)), device="cuda")
    _sampled(B, w, rows)


def test_batched_matches_per_matrix(B):
    x = W.random_matrix(5 * 48, 96, seed=8, dtype=torch.bfloat16, device="cuda").reshape(5, 48, 96)
    x[2] *= 100.0
    x[4] = 0.0
    q, s, g = B.nvfp4_quantize_batched(x.contiguous())
    for b in range(5):
        rq, rs, rg = Q.quantize(_host(x[b]))
        assert g[b].item() == rg, b
        np.testing.assert_array_equal(s[b].cpu().numpy(), rs)
        np.testing.assert_array_equal(q[b].cpu().numpy(), rq)


def test_deterministic(B):
    x, _ = W.linear_inputs("prefill_8192x5120", device="cuda", M=512)
    a = B.nvfp4_quantize(x)
    b = B.nvfp4_quantize(x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def _barrier_timeouts(B):
    """Expired-wait counter of the single-read kernel in every cached workspace (0 when healthy)."""
    torch.cuda.synchronize()
    return sum(int(ws[8:12].view(torch.int32).item()) for ws in B._QWS.values())


def test_midpoint_sweep_exact_scaling(B):
    """Blocks whose scale makes r = 1, so y = x: codes follow E2M1 rounding directly.

    Row 0 holds 2688 (g = 1); every other block holds a 6 (scale 1.0, r = 1)
    and 15 values at, or a few float32 ulps around, grid points and midpoints.
    """
    vals = []
    for m in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]:
        for sgn in (1.0, -1.0):
            v = np.float32(m * sgn)
            vals.append(v)
            up = dn = v
            for _ in range(3):
                up = np.nextafter(up, np.float32(np.inf), dtype=np.float32)
                dn = np.nextafter(dn, np.float32(-np.inf), dtype=np.float32)
                vals += [up, dn]
    vals += [np.float32(0.0), np.float32(-0.0), np.float32(1e-30), np.float32(-1e-30),
             np.float32(5.999999), np.float32(-5.9999995)]
    vals = [v for v in vals if abs(v) <= 6.0]
    nblk = -(-len(vals) // 15)
    vals += [np.float32(0.0)] * (nblk * 15 - len(vals))
    blocks = np.array(vals, dtype=np.float32).reshape(nblk, 15)
    body = np.concatenate([np.full((nblk, 1), 6.0, np.float32), blocks], axis=1).reshape(1, -1)
    head = np.zeros((1, body.shape[1]), np.float32)
    head[0, 0] = 2688.0
    x = np.concatenate([head, body])
    for dt in (torch.float32, torch.bfloat16):
        xt = torch.from_numpy(x).cuda().to(dt)
        if dt == torch.bfloat16 and not np.array_equal(xt.float().cpu().numpy(), x):
            xt = torch.from_numpy(x).cuda()  # values not bf16-exact: sweep in fp32 only
        _check_full(B, xt)
        rq, rs, rg = Q.quantize(x)
        assert rg == 1.0 and np.all(rs[1] == 0x38)


def test_two_pass_path_large_bf16(B):
    """More blocks than the register file holds: the amax + encode passes."""
    x = W.random_matrix(8192, 6144, seed=21, dtype=torch.bfloat16, device="cuda")
    print("[quantize] two-pass 8192x6144 bf16", flush=True)
    rows = torch.tensor([0, 1, 4097, 8191] + list(range(5, 8192, 509)), device="cuda")
    _sampled(B, x, rows)


def test_fp32_moe_h_two_pass(B):
    """float32 h of the 128-expert MoE (32768 x 768): 1.2 times what the
    single-read path holds (10 float32 blocks per thread), so the two-pass path."""
    x = W.random_matrix(32768, 768, seed=22, device="cuda")
    rows = torch.tensor([0, 32767] + list(range(3, 32768, 1021)), device="cuda")
    _sampled(B, x, rows)


def test_many_calls_reuse_the_workspace(B):
    before = _barrier_timeouts(B)
    for i, (r, c) in enumerate([(4096, 2048), (1, 16), (8192, 5120), (3, 48), (2000, 4096)] * 4):
        x = W.random_matrix(r, c, seed=100 + i, dtype=torch.bfloat16, device="cuda") * (1.0 + i)
        q, s, g = B.nvfp4_quantize(x)
        assert g.item() == Q.global_scale(_host(x)), (i, r, c)
        rr = torch.tensor([0, r - 1], device="cuda")
        rq, rs, _ = Q.quantize(_host(x[rr]), g=g.item())
        np.testing.assert_array_equal(s[rr].cpu().numpy(), rs)
        np.testing.assert_array_equal(q[rr].cpu().numpy(), rq)
    assert _barrier_timeouts(B) == before == 0


def test_expired_waits_take_the_whole_tensor_max(B):
    """The single-read kernel's bounded arrival wait, forced to expire from the
    host: word 3 of the workspace's arrival state holds a wait bound in polls (0:
    the built-in bound) that the kernels never write.  At one poll most
    workgroups stop waiting and read the whole tensor for the max themselves;
    codes, scales and the global scale stay bit-exact, the expired waits are
    counted (word 2), and a call with the built-in bound then runs on the same
    workspace.  Called through the C-ABI with a workspace of the test's own."""
    lib = B.load_library()
    rows, cols = 1024, 2048
    ws = torch.zeros(int(lib.nvfp4_quantize_workspace_size(rows, cols)), dtype=torch.uint8, device="cuda")
    words = ws[:16].view(torch.int32)
    for i, bound in enumerate([1, 1, 0]):
        print(f"[quantize] wait bound {bound}, call {i}", flush=True)
        x = W.random_matrix(rows, cols, seed=300 + i, dtype=torch.bfloat16, device="cuda") * (1.0 + i)
        words[3] = bound
        words[2] = 0
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda")
        g = torch.empty(1, dtype=torch.float32, device="cuda")
        st = lib.nvfp4_quantize(B._ptr(x), B.NVFP4_BF16, rows, cols, cols, B._ptr(q), B._ptr(s), B._ptr(g), 0,
                                B._ptr(ws), ws.numel(), B._stream())
        assert st == 0
        torch.cuda.synchronize()
        rq, rs, rg = Q.quantize(_host(x))
        assert g.item() == rg, i
        np.testing.assert_array_equal(s.cpu().numpy(), rs)
        np.testing.assert_array_equal(q.cpu().numpy(), rq)
        if bound:
            assert int(words[2].item()) > 0, "no wait expired at a bound of one poll"


def test_concurrent_streams_stay_exact(B):
    """Dynamic quantizes of two tensors issued on two streams at once (default
    priority, one cached workspace each): the single-read kernels share the
    compute units, so a workgroup may wait past its bound and read the whole
    tensor for the max; codes, scales and global scales stay exact either way."""
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xs = [W.random_matrix(4096, 5120, seed=400 + i, dtype=torch.bfloat16, device="cuda") * (1.0 + 3 * i)
          for i in range(2)]
    torch.cuda.synchronize()
    outs = []
    for it in range(3):
        print(f"[quantize] two streams, round {it}", flush=True)
        with torch.cuda.stream(s1):
            r1 = B.nvfp4_quantize(xs[0])
        with torch.cuda.stream(s2):
            r2 = B.nvfp4_quantize(xs[1])
        outs.append((r1, r2))
    torch.cuda.synchronize()
    keys = [k for k in B._QWS if k[1] in (s1.cuda_stream, s2.cuda_stream)]
    waits = sum(int(B._QWS[k][8:12].view(torch.int32).item()) for k in keys)
    print(f"[quantize] two streams: {waits} expired waits", flush=True)
    for x, i in zip(xs, range(2)):
        xh = _host(x)
        rg = Q.global_scale(xh)
        rows = np.array([0, 1, 4095] + list(range(7, 4096, 331)))
        rq, rs, _ = Q.quantize(xh[rows], g=rg)
        for pair in outs:
            q, s, g = pair[i]
            assert g.item() == rg
            sel = torch.as_tensor(rows, device="cuda")
            np.testing.assert_array_equal(s[sel].cpu().numpy(), rs)
            np.testing.assert_array_equal(q[sel].cpu().numpy(), rq)
    for k in keys:  # these workspaces were only for this test
        del B._QWS[k]


def test_explicit_stream_not_current(B):
    """stream= names a stream that is not torch's current one: the workspace is
    allocated and zero-filled on that stream, so the first launch there sees the
    fill; a larger tensor then grows the workspace on the same stream.  Codes,
    scales and global scales bit-exact against the oracle."""
    s = torch.cuda.Stream()
    xs = [W.random_matrix(r, c, seed=500 + r, dtype=torch.bfloat16, device="cuda") * (2.0 + r)
          for r, c in [(64, 256), (4096, 4096), (300, 1024)]]
    torch.cuda.synchronize()
    outs = []
    for x in xs:
        print(f"[quantize] explicit stream {tuple(x.shape)}", flush=True)
        with torch.cuda.stream(s):
            qo = (torch.empty((x.shape[0], x.shape[1] // 2), dtype=torch.uint8, device="cuda"),
                  torch.empty((x.shape[0], x.shape[1] // 16), dtype=torch.uint8, device="cuda"),
                  torch.empty(1, dtype=torch.float32, device="cuda"))
        outs.append(B.nvfp4_quantize(x, out=qo, stream=s))
    s.synchronize()
    for x, (q, sc, g) in zip(xs, outs):
        rq, rs, rg = Q.quantize(_host(x))
        assert g.item() == rg
        np.testing.assert_array_equal(sc.cpu().numpy(), rs)
        np.testing.assert_array_equal(q.cpu().numpy(), rq)
    key = (torch.cuda.current_device(), int(s.cuda_stream))
    assert int(B._QWS[key][8:12].view(torch.int32).item()) == 0  # no expired waits
    del B._QWS[key]
