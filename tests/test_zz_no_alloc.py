"""The allocation-free quantize entry point (nvfp4_quantize_noalloc), called
through the C ABI, against nvfp4_quantize with a workspace of its own.

Bar: codes, scales and global scales bit-identical to the existing entry
point's.  Two calls in a row on the same stream, the second with a smaller
input, so the second reuses the per-GPU scratch the first left behind: the
first takes the two-pass path (more blocks than the register file holds: its
amax partials live in the scratch), the second the single-read path (its
arrival state lives there); then the same again in float32, and a static
global scale.  Under HIP graph capture: replays of a captured call match the
entry point on each replay's input.
"""

import numpy as np
import pytest
import torch

from moe_nvfp4_quantize_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from moe_nvfp4_quantize_amd import nvfp4
    nvfp4.load_library()
    return nvfp4


def _noalloc_abi(B, x, g=None):
    """Direct C-ABI call of nvfp4_quantize_noalloc with outputs of the test's own."""
    lib = B.load_library()
    rows, cols = x.shape
    q = torch.full((rows, cols // 2), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, cols // 16), 0xA5, dtype=torch.uint8, device="cuda")
    gg = torch.full((1,), -1.0, dtype=torch.float32, device="cuda") if g is None else g.clone()
    st = lib.nvfp4_quantize_noalloc(B._ptr(x), B._dtype_code(x.dtype), rows, cols, x.stride(0),
                                    B._ptr(q), B._ptr(s), B._ptr(gg), int(g is not None), B._stream())
    assert st == B.NVFP4_OK, B.status_string(st)
    return q, s, gg


def _same(a, b, label):
    torch.cuda.synchronize()
    for u, v, name in zip(a, b, "qsg"):
        assert torch.equal(u, v), (label, name)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_entry_point(B, dtype):
    big = (8192, 6144) if dtype == torch.bfloat16 else (4096, 6144)   # two-pass path
    small = (1000, 2048)                                              # single-read path
    for i, (r, c) in enumerate([big, small]):
        print(f"[noalloc] call {i}: {r}x{c} {dtype}", flush=True)
        x = W.random_matrix(r, c, seed=900 + i, dtype=dtype, device="cuda") * (1.0 + 5 * i)
        got = _noalloc_abi(B, x)
        want = B.nvfp4_quantize(x)
        _same(got, want, (i, r, c))
        assert got[2].item() > 0


def test_noalloc_static_scale_and_repeats(B):
    x = W.random_matrix(512, 4096, seed=950, dtype=torch.bfloat16, device="cuda")
    g = torch.tensor([0.01], dtype=torch.float32, device="cuda")
    _same(_noalloc_abi(B, x, g), B.nvfp4_quantize(x, g=g), "static")
    for i in range(3):  # the arrival state left by each call serves the next
        xi = x[: 512 - 100 * i] * (i + 1.0)
        _same(_noalloc_abi(B, xi), B.nvfp4_quantize(xi), ("repeat", i))


@pytest.mark.parametrize("shape", [(1000, 2048), (8192, 6144)])  # single-read, two-pass path
def test_noalloc_under_graph_capture(B, shape):
    """Captured in a HIP graph (the callers it serves) after one eager call has
    set up the GPU's scratch, then replayed three times with the input rewritten
    in place and eager work between the replays (the workspace entry point on
    the same input): every replay bit-identical to that entry point."""
    r, c = shape
    x = W.random_matrix(r, c, seed=960, dtype=torch.bfloat16, device="cuda")
    q = torch.empty((r, c // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((r, c // 16), dtype=torch.uint8, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    B.nvfp4_quantize_noalloc(x, out=(q, s, g))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.nvfp4_quantize_noalloc(x, out=(q, s, g))
    torch.cuda.synchronize()
    for i in range(3):
        print(f"[noalloc] graph replay {i}: {r}x{c} bf16", flush=True)
        x.copy_(W.random_matrix(r, c, seed=961 + i, dtype=torch.bfloat16, device="cuda") * (1.0 + 3 * i))
        want = B.nvfp4_quantize(x)
        graph.replay()
        _same((q, s, g), want, ("replay", i, shape))


def test_noalloc_rejects_invalid(B):
    lib = B.load_library()
    fake = B.ctypes.c_void_p(0x1000)
    assert lib.nvfp4_quantize_noalloc(fake, B.NVFP4_BF16, 4, 24, 24, fake, fake, fake, 0, None) == \
        B.NVFP4_ERR_INVALID_ARG
    assert lib.nvfp4_quantize_noalloc(fake, B.NVFP4_BF16, 4, 32, 32, fake, fake, None, 0, None) == \
        B.NVFP4_ERR_INVALID_ARG
