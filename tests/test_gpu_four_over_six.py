"""GPU parity of nvfp4_quantize_4over6 against the four-over-six oracle:
codes, block scales and global scales bit-exact."""

import numpy as np
import pytest
import torch

from oracle import four_over_six as F
from oracle import nvfp4 as Q
from moe_nvfp4_quantize_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from moe_nvfp4_quantize_amd import nvfp4
    nvfp4.load_library()
    return nvfp4


def _check(B, x_dev, label):
    q, s, g = B.nvfp4_quantize_4over6(x_dev)
    torch.cuda.synchronize()
    xh = x_dev.float().cpu().numpy()
    rq, rs, rg, took4 = F.quantize(xh)
    assert np.float32(g.item()) == rg, label
    np.testing.assert_array_equal(s.cpu().numpy(), rs, err_msg=label)
    np.testing.assert_array_equal(q.cpu().numpy(), rq, err_msg=label)
    print(f"[4/6] {label}: bit-exact, {took4.mean():.1%} of blocks take M = 4", flush=True)
    return took4


def test_linear_16x512_weights(B):
    _, w = W.linear_inputs("linear_16x512", device="cuda")
    took4 = _check(B, w, "W f32 256x512")
    assert 0.05 < took4.mean() < 0.95


@pytest.mark.parametrize("rows,cols,dtype", [(300, 1024, torch.bfloat16), (7, 48, torch.float32),
                                             (1, 16, torch.bfloat16), (129, 272, torch.float32)])
def test_random(B, rows, cols, dtype):
    x = W.random_matrix(rows, cols, seed=rows + cols, dtype=dtype, device="cuda", std=0.02)
    _check(B, x, f"{rows}x{cols} {dtype}")


def test_hand_built_blocks(B):
    four = [4, 3, 2, 1.5, 1, 0.5, 0, -4, -3, -2, -1.5, -1, -0.5, 0, 3, 2]
    six = [6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, -2, -1.5, -1, -0.5, 0]
    x = np.zeros((2, 48), dtype=np.float32)
    x[0, :16], x[0, 16:32], x[0, 32] = four, six, 168.0
    x[1, 40] = -3.0  # a zero block, a block with one value
    took4 = _check(B, torch.from_numpy(x).cuda(), "hand-built blocks")
    assert took4[0].tolist() == [True, False, False]


def test_batched_experts(B):
    x = torch.stack([W.random_matrix(64, 256, seed=100 + e, device="cuda", std=0.02 * (e + 1))
                     for e in range(3)]).to(torch.bfloat16).contiguous()
    q, s, g = B.nvfp4_quantize_4over6(x)
    torch.cuda.synchronize()
    for e in range(3):
        rq, rs, rg, _ = F.quantize(x[e].float().cpu().numpy())
        assert np.float32(g[e].item()) == rg
        np.testing.assert_array_equal(s[e].cpu().numpy(), rs)
        np.testing.assert_array_equal(q[e].cpu().numpy(), rq)


def test_prefill_weights_sampled_rows(B):
    _, w = W.linear_inputs("prefill_8192x5120", device="cuda")
    q, s, g = B.nvfp4_quantize_4over6(w)
    torch.cuda.synchronize()
    wh = w.float().cpu().numpy()
    rg = Q.global_scale(wh)
    assert np.float32(g.item()) == rg
    rows = np.array([0, 1, 12799, 25599] + list(range(5, 25600, 997)))
    rq, rs, _, _ = F.quantize(wh[rows], g=rg)
    np.testing.assert_array_equal(s.cpu().numpy()[rows], rs)
    np.testing.assert_array_equal(q.cpu().numpy()[rows], rq)
