"""Seeded synthetic inputs for the five NVFP4 workloads.

This module only draws random tensors: it holds none of the quantization, GEMM
or routing arithmetic, and both the GPU path and the CPU oracle are fed from it.

The pages measure on trained checkpoints, calibration sets and serving
benchmarks; none is available offline, so seeded tensors with the shapes and
value distributions below stand in for them:

  linear_16x512      X fp32 [16, 512] ~ N(0, 1) with 1% of entries (82, drawn
                     without replacement) multiplied by 20; W fp32 [256, 512]
                     ~ N(0, 0.02^2); Y = X W^T fp32.                   seed 0
  prefill_8192x5120  X bf16 [8192, 5120] = Z * c[col], Z ~ N(0,1), per input
                     channel c ~ LogNormal(0, 1); W bf16 [25600, 5120]
                     ~ N(0, 0.02^2); bf16 out.                          seed 1
  lmhead_128x151936  X bf16 [128, 2048] ~ N(0,1); W bf16 [151936, 2048]
                     ~ N(0, 0.02^2), quantized once offline; bf16 out.  seed 2
  moe_e128_top8      router logits fp32 [4096, 128] ~ N(0,1); X bf16 [4096, 2048]
                     ~ N(0,1); gate_up bf16 [128, 1536, 2048] and down bf16
                     [128, 2048, 768] ~ N(0, 0.02^2); k = 8.            seed 3
  moe_e512_top10     as above with T=8192, E=512, H=4096, I=1024, k=10, plus a
                     hot-expert skew: 16 hot experts and round(0.1*T) tokens
                     drawn from the seed, those tokens' logits at the hot
                     experts raised by 4.0.                             seed 4

All draws use ``torch.Generator`` on the device the tensors are made on, so a
test that checks a GPU result copies the same tensors to the host for the
oracle; nothing is regenerated on another device.
"""

import torch

WORKLOADS = {
    "linear_16x512": dict(kind="linear", M=16, N=256, K=512, x_dtype="f32", out="f32", seed=0),
    "prefill_8192x5120": dict(kind="linear", M=8192, N=25600, K=5120, x_dtype="bf16", out="bf16", seed=1),
    "lmhead_128x151936": dict(kind="linear", M=128, N=151936, K=2048, x_dtype="bf16", out="bf16", seed=2),
    "moe_e128_top8": dict(kind="moe", T=4096, E=128, k=8, H=2048, I=768, seed=3, hot=0),
    "moe_e512_top10": dict(kind="moe", T=8192, E=512, k=10, H=4096, I=1024, seed=4, hot=16),
}

W_STD = 0.02


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def calibration_rows(name, rows, device="cpu"):
    """Activations of a dense workload's layer for calibrating a static global
    scale: ``rows`` fresh rows (their own seed) under the workload's fixed
    per-channel scales, so they follow the same distribution as X."""
    cfg = WORKLOADS[name]
    K = cfg["K"]
    if name == "prefill_8192x5120":
        # the channel scales c are drawn after Z in the workload's own stream
        gen = _gen(cfg["seed"], device)
        _normal((cfg["M"], K), 1.0, gen, device)
        c = torch.exp(_normal((K,), 1.0, gen, device))
        z = _normal((rows, K), 1.0, _gen(cfg["seed"] + 1000, device), device)
        return (z * c[None, :]).to(torch.bfloat16)
    dtype = torch.float32 if cfg["x_dtype"] == "f32" else torch.bfloat16
    return _normal((rows, K), 1.0, _gen(cfg["seed"] + 1000, device), device).to(dtype)


def moe_calibration_inputs(name, T, device="cpu"):
    """(logits, X) of ``T`` fresh tokens (their own seed) for an MoE workload:
    the batch a static activation scale is calibrated on."""
    cfg = WORKLOADS[name]
    gen = _gen(cfg["seed"] + 1000, device)
    logits = _normal((T, cfg["E"]), 1.0, gen, device)
    x = _normal((T, cfg["H"]), 1.0, gen, device).to(torch.bfloat16)
    return logits, x


def linear_inputs(name, device="cpu", M=None):
    """(X, W) for a dense workload; ``M`` overrides the row count of X."""
    cfg = WORKLOADS[name]
    M = cfg["M"] if M is None else M
    N, K = cfg["N"], cfg["K"]
    gen = _gen(cfg["seed"], device)
    if name == "linear_16x512":
        x = _normal((M, K), 1.0, gen, device)
        n_out = int(round(0.01 * M * K))
        idx = torch.randperm(M * K, generator=gen, device=device)[:n_out]
        flat = x.reshape(-1)
        flat[idx] = flat[idx] * 20.0
        w = _normal((N, K), W_STD, gen, device)
        return x, w
    if name == "prefill_8192x5120":
        z = _normal((M, K), 1.0, gen, device)
        c = torch.exp(_normal((K,), 1.0, gen, device))
        x = (z * c[None, :]).to(torch.bfloat16)
        w = _normal((N, K), W_STD, gen, device).to(torch.bfloat16)
        return x, w
    if name == "lmhead_128x151936":
        x = _normal((M, K), 1.0, gen, device).to(torch.bfloat16)
        w = _normal((N, K), W_STD, gen, device).to(torch.bfloat16)
        return x, w
    raise KeyError(name)


def moe_inputs(name, device="cpu", T=None, E=None, H=None, I=None, k=None, hot=None, weights=True):
    """dict(logits, x, w_gate_up, w_down, k) for an MoE workload; sizes overridable.
    ``weights=False`` stops after X (same logits and X; no expert weights)."""
    cfg = dict(WORKLOADS[name])
    for key, val in dict(T=T, E=E, H=H, I=I, k=k, hot=hot).items():
        if val is not None:
            cfg[key] = val
    T, E, H, I, k = cfg["T"], cfg["E"], cfg["H"], cfg["I"], cfg["k"]
    gen = _gen(cfg["seed"], device)
    logits = _normal((T, E), 1.0, gen, device)
    if cfg["hot"]:
        hot_ids = torch.randperm(E, generator=gen, device=device)[: cfg["hot"]]
        n_tok = int(round(0.1 * T))
        toks = torch.randperm(T, generator=gen, device=device)[:n_tok]
        logits[toks[:, None], hot_ids[None, :]] += 4.0
    x = _normal((T, H), 1.0, gen, device).to(torch.bfloat16)
    if not weights:
        return dict(logits=logits, x=x, k=k)
    w_gu = torch.empty((E, 2 * I, H), dtype=torch.bfloat16, device=device)
    w_d = torch.empty((E, H, I), dtype=torch.bfloat16, device=device)
    # one expert at a time keeps the float32 temporaries small
    for e in range(E):
        w_gu[e] = _normal((2 * I, H), W_STD, gen, device).to(torch.bfloat16)
    for e in range(E):
        w_d[e] = _normal((H, I), W_STD, gen, device).to(torch.bfloat16)
    return dict(logits=logits, x=x, w_gate_up=w_gu, w_down=w_d, k=k)


def random_matrix(rows, cols, seed, dtype=torch.float32, device="cpu", std=1.0):
    """A plain N(0, std^2) matrix for edge-case tests."""
    gen = _gen(seed, device)
    return _normal((rows, cols), std, gen, device).to(dtype)


def ceil_div(a, b):
    return -(-a // b)


def describe(name):
    cfg = WORKLOADS[name]
    return name + ": " + ", ".join(f"{k}={v}" for k, v in cfg.items())
