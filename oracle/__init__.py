"""CPU oracle for the NVFP4 W4A4 hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
restatement of what the NVFP4 quantized linear layer and its routed-expert MoE
variant compute.  Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it.  The GPU library never calls into it, and it
imports nothing from the GPU library.

Sources (a reader has the pages, not a copy of them):

* Qwen3.8-Flash-Next-NVFP4 page ("How is the NVFP4 quantization of
  Qwen3.8-Flash-Next-NVFP4 done? W4A4 two-level scaling and why only routed
  experts are quantized", bjdmk.com.cn), referred to below as the *two-level
  scaling page*:
    - section "Core: the W4A4 two-level scaling mechanism", level 1 (16-element
      blocks along the last dimension, one E4M3 block scale each, E2M1 elements)
      and level 2 (one FP32 global scale per tensor; scale audit: all scales
      finite and positive, min about 2.13e-05, max 448.0);
    - the shard metadata recipe quoted in that section (num_bits [2,1],
      block size 16 on dim -1, scale_bits [4,3], type dynamic,
      effective_bits 4.5);
    - sub-section "Why 4.5 bits" ((16*4 + 8)/16 = 4.5);
    - sub-section "The A4 side: dynamic activations" (weights static,
      activations quantized on the fly with the same 16-block rule);
    - section "Why only routed experts" (top-10 of 512 routed experts per token,
      router kept in BF16).
* Model-Optimizer QAD tutorial for Qwen3.6-35B-A3B W4A4 NVFP4 (pwwt.cn), section
  "Why W4A4 rather than W4A16" (both operands in FP4 so the GEMM runs on the
  FP4 units; lm_head included).

Where the pages leave a step open, the oracle takes the reading recorded in the
repository's design notes; each such reading is named where it is used.

Modules:
    formats  -- E2M1 and E4M3 decode / round-to-nearest-even encode
    nvfp4    -- two-level quantize and dequantize
    gemm     -- the W4A4 GEMM as an fp64 product of dequantized operands
    moe      -- router top-k + softmax, permutation, expert MLP, combine
    four_over_six -- weight block scales chosen between maps to 6 and to 4
    qdq      -- quantize then dequantize (fake quantization)
    fp8      -- FP8 E4M3 per-tensor W8A8 quantize, dequantize and GEMM
"""

from . import formats, nvfp4, gemm, moe  # noqa: F401
