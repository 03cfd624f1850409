"""GPU parity of nvfp4_qdq (quantize-dequantize) against the oracle: every
output value bit-exact, dynamic and frozen global scales, both dtypes, the
single-read and two-pass paths, in place."""

import numpy as np
import pytest
import torch

from oracle import nvfp4 as Q
from oracle import qdq as D
from moe_nvfp4_quantize_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from moe_nvfp4_quantize_amd import nvfp4
    nvfp4.load_library()
    return nvfp4


def _out(x):
    return "bf16" if x.dtype == torch.bfloat16 else "f32"


def _check(B, x, g=None, label=""):
    y, gg = B.nvfp4_qdq(x, g=g)
    torch.cuda.synchronize()
    xh = x.float().cpu().numpy()
    ref, rg = D.qdq(xh, g=None if g is None else np.float32(g.item()), out=_out(x))
    assert np.float32(gg.item()) == rg
    np.testing.assert_array_equal(y.float().cpu().numpy(), ref, err_msg=label)
    return y


def test_linear_16x512_dynamic(B):
    x, _ = W.linear_inputs("linear_16x512", device="cuda")
    _check(B, x, label="C1 X")


@pytest.mark.parametrize("rows,cols,dtype", [(300, 1024, torch.bfloat16), (7, 48, torch.float32),
                                             (1, 16, torch.bfloat16), (129, 272, torch.float32),
                                             (65, 4096, torch.bfloat16)])
def test_random_dynamic(B, rows, cols, dtype):
    x = W.random_matrix(rows, cols, seed=rows * 3 + cols, dtype=dtype, device="cuda")
    _check(B, x, label=f"{rows}x{cols}")


def test_frozen_scale_saturates(B):
    x = W.random_matrix(64, 512, seed=9, dtype=torch.bfloat16, device="cuda")
    g = torch.tensor([float(Q.global_scale(x.float().cpu().numpy())) / 8], device="cuda")
    _check(B, x, g=g, label="frozen g / 8")


def test_in_place_and_strided(B):
    x = W.random_matrix(40, 256, seed=4, device="cuda")
    ref, _ = D.qdq(x.cpu().numpy())
    B.nvfp4_qdq(x, out=x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(x.cpu().numpy(), ref)
    big = W.random_matrix(40, 320, seed=5, dtype=torch.bfloat16, device="cuda")
    view = big[:, :256]
    ref2, _ = D.qdq(view.float().cpu().numpy(), out="bf16")
    y, _ = B.nvfp4_qdq(view)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.float().cpu().numpy(), ref2)


def test_prefill_activations_sampled_rows(B):
    x, _ = W.linear_inputs("prefill_8192x5120", device="cuda")
    y, g = B.nvfp4_qdq(x)
    torch.cuda.synchronize()
    xh = x.float().cpu().numpy()
    rg = Q.global_scale(xh)
    assert np.float32(g.item()) == rg
    rows = np.array([0, 1, 4095, 8191] + list(range(7, 8192, 331)))
    ref, _ = D.qdq(xh[rows], g=rg, out="bf16")
    np.testing.assert_array_equal(y[torch.as_tensor(rows, device="cuda")].float().cpu().numpy(), ref)


def test_two_pass_path_sampled_rows(B):
    # 25600 x 5120 bf16 is beyond the single-read kernel's register capacity
    _, w = W.linear_inputs("prefill_8192x5120", device="cuda")
    y, g = B.nvfp4_qdq(w)
    torch.cuda.synchronize()
    wh = w.float().cpu().numpy()
    rg = Q.global_scale(wh)
    assert np.float32(g.item()) == rg
    rows = np.array([0, 25599] + list(range(13, 25600, 1409)))
    ref, _ = D.qdq(wh[rows], g=rg, out="bf16")
    np.testing.assert_array_equal(y[torch.as_tensor(rows, device="cuda")].float().cpu().numpy(), ref)
