/*
 * nvfp4.h -- C ABI of libnvfp4.so: NVFP4 W4A4 quantize, GEMM and routed-expert
 * MoE kernels for AMD Instinct MI355X (gfx950).
 *
 * Format (Qwen3.8-Flash-Next-NVFP4 page, section "Core: the W4A4 two-level
 * scaling mechanism"): a tensor [rows x cols] is cut into 16-element blocks
 * along cols (its last dimension).  Each element is a 4-bit E2M1 code, each
 * block has one E4M3 (E4M3FN, largest value 448) scale, and the tensor has one
 * FP32 global scale; (16*4 + 8)/16 = 4.5 bits per element ("Why 4.5 bits").
 *
 * An NVFP4 tensor at this ABI is three device buffers:
 *   q  uint8 [rows][cols/2]   two codes per byte, element 2j in bits 3..0 and
 *                             element 2j+1 in bits 7..4; code bit 3 is the sign
 *   s  uint8 [rows][cols/16]  E4M3FN scale codes, row-major, always positive
 *   g  float [1]              decode multiplier: x_hat = e2m1(q) * e4m3(s) * g
 * Rows of q and s are dense (row strides cols/2 and cols/16 bytes).
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer unless its comment says host.
 *     The caller owns all memory; the library never allocates or frees device
 *     memory and never synchronizes: each call validates its arguments on the
 *     host, enqueues kernels on `stream` and returns.
 *   - Arguments are validated before any HIP call.  On failure the call returns
 *     NVFP4_ERR_INVALID_ARG (or NVFP4_ERR_UNSUPPORTED for a valid request this
 *     build does not implement) and touches no device memory.
 *   - A failed launch returns NVFP4_ERR_HIP; the HIP error is not cleared.
 *   - The current HIP device must be a gfx950 GPU, otherwise
 *     NVFP4_ERR_UNSUPPORTED is returned.
 *   - Inputs must be finite; non-finite inputs give unspecified (but in-bounds)
 *     results.  Nothing is printed and nothing aborts.
 *   - Calls on one stream are ordered; calls that share output or workspace
 *     buffers on different streams race.  The library keeps no global state
 *     other than per-device caches of the architecture check and the compute
 *     unit count, and the per-GPU scratch array of nvfp4_quantize_noalloc.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1,
  NVFP4_ERR_UNSUPPORTED = 2,
  NVFP4_ERR_HIP = 3
} nvfp4_status;

typedef enum {
  NVFP4_F32 = 0,  /* IEEE binary32 */
  NVFP4_BF16 = 1  /* bfloat16; results are rounded to nearest even */
} nvfp4_dtype;

/* Version of this ABI (bumped on any incompatible change). */
#define NVFP4_ABI_VERSION 1
int nvfp4_abi_version(void);

/* Static, human-readable name of a status code (host). */
const char *nvfp4_status_string(nvfp4_status status);

/* ------------------------------------------------------------------------
 * Quantize (two-level scaling page: level 1 block scales, level 2 global
 * scale; sub-section "The A4 side: dynamic activations").
 *
 * x       [rows][ld_x] of x_type (f32 or bf16), quantized along its first
 *         `cols` columns; ld_x >= cols, in elements.
 * rows    >= 0 (0 is a no-op apart from the global scale, see below)
 * cols    > 0 and a multiple of 16
 * q, s    outputs as described at the top of this file
 * g       device float.  static_global == 0 (dynamic): written with
 *         g = amax/2688 (amax = max|x|; 2688 = 6*448), or 1.0 when amax == 0.
 *         static_global != 0: read as the caller's global scale (a positive
 *         normal float >= 2^-100), not written.
 * Per block (all float32, round to nearest even):
 *   s = E4M3(min(bmax / (6*g), 448)), raised to 2^-9 if it rounds to 0;
 *   r = 1 / (s*g);  code = E2M1(min(|x*r|, 6)) with the sign of x.
 * workspace  device scratch of at least nvfp4_quantize_workspace_size(rows,
 *         cols) bytes, 256-byte aligned (dynamic mode only; may be NULL when
 *         static_global != 0).  It must be zero-filled before its first use
 *         and then be left to this function: its first bytes hold the arrival
 *         state of the single-read kernel, which every completed call leaves
 *         ready for the next.  One workspace may serve any number of calls in
 *         stream order; calls that overlap in time (different streams) need
 *         separate workspaces.
 * Dynamic mode reads x once from HBM when it fits in the register file of the
 * GPU (about 42 M bf16 / 21 M fp32 elements on 256 CUs): one workgroup per CU
 * keeps its share in registers while the workgroups exchange their maxima.
 * If the workgroups are not all resident at once (other work occupying CUs),
 * a workgroup whose bounded wait expires reads the whole tensor for the max
 * itself: slower, same result.  Larger tensors take a two-pass path (amax,
 * encode).
 * Precondition for the dynamic mode: amax == 0 or amax >= 2^-100.
 * Alignment: x 16-byte aligned and ld_x*elem_size a multiple of 16 for the
 * vectorised path; other layouts are accepted and take a slower path.
 * ---------------------------------------------------------------------- */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols);
nvfp4_status nvfp4_quantize(const void *x, nvfp4_dtype x_type, int64_t rows,
                            int64_t cols, int64_t ld_x, uint8_t *q, uint8_t *s,
                            float *g, int static_global, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* nvfp4_quantize without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * nvfp4_quantize; the scratch the dynamic mode needs (the single-read
 * kernel's arrival state and at most 256 amax partials: 9472 bytes) is a
 * device array inside the library, one per GPU, held until the process ends,
 * so every shape nvfp4_quantize accepts fits (a request that would need more
 * returns NVFP4_ERR_INVALID_ARG).  Nothing is allocated: the first call on a
 * device looks up that device's copy of the array and zero-fills it with a
 * kernel on `stream`; every completed call leaves it ready for the next.
 * All calls on one GPU share that array: calls that overlap in time on one
 * GPU (different streams, or host threads) race and may return wrong global
 * scales; serialize them, or use nvfp4_quantize with separate workspaces. */
nvfp4_status nvfp4_quantize_noalloc(const void *x, nvfp4_dtype x_type,
                                    int64_t rows, int64_t cols, int64_t ld_x,
                                    uint8_t *q, uint8_t *s, float *g,
                                    int static_global, hipStream_t stream);

/* Batched dynamic quantize of `batch` independent matrices laid out
 * contiguously: x [batch][rows][cols] (dense), q [batch][rows][cols/2],
 * s [batch][rows][cols/16], g [batch]; matrix b gets its own global scale
 * g[b] = amax_b/2688.  This is the offline (static) weight quantization of the
 * per-expert matrices of an MoE (two-level scaling page, sub-section "The A4
 * side": weights are quantized offline; one global scale per tensor).
 * workspace: nvfp4_quantize_batched_workspace_size(batch, rows, cols) bytes,
 * 4-byte aligned; its contents on entry do not matter (it is clobbered). */
size_t nvfp4_quantize_batched_workspace_size(int64_t batch, int64_t rows,
                                             int64_t cols);
nvfp4_status nvfp4_quantize_batched(const void *x, nvfp4_dtype x_type,
                                    int64_t batch, int64_t rows, int64_t cols,
                                    uint8_t *q, uint8_t *s, float *g,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * Quantize-dequantize ("fake quantization"), the simulated-quantization
 * forward of quantization-aware distillation (QAD page: NVFP4 simulated in
 * the forward pass, with scales either recomputed every step -- dynamic -- or
 * calibrated once and frozen -- static_global != 0).
 *
 * y[r][c] = fl(e2m1(code) * e4m3(s) * g) for the codes and block scales that
 * nvfp4_quantize computes from x with the same rows, cols, g and mode; the
 * product e2m1 * e4m3 is exact, the multiplication by g rounds once to float32
 * and a bf16 y rounds that once more (nearest even).  y has x's type, row
 * stride ld_y >= cols (elements); y may be x itself (in place) when
 * ld_y == ld_x.  g, static_global, workspace: as for nvfp4_quantize (the
 * dynamic g is written).  No codes or scales are stored.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_qdq(const void *x, nvfp4_dtype x_type, int64_t rows,
                       int64_t cols, int64_t ld_x, void *y, int64_t ld_y,
                       float *g, int static_global, void *workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Offline (weight) quantize with four-over-six block scales (Nemotron 3.5
 * Lightning QAD page, PTQ recipe table: "4/6", the block maximum mapped to
 * E2M1 magnitude 6 or 4, whichever gives the lower squared error; such
 * searched scales are then kept frozen).
 *
 * Same layout, global scale (g[b] = amax_b/2688 per matrix) and workspace as
 * nvfp4_quantize_batched; for every block both candidates are encoded:
 *   M = 6: s6 = E4M3(min(bmax/(6*g), 448)), the plain scale;
 *   M = 4: s4 = E4M3(min(bmax/(4*g), 448));   (a zero raised to 2^-9)
 * codes from r = 1/(s*g) as in nvfp4_quantize, and the block keeps M = 4 iff
 * its float32 error sum E4 < E6, where E = sum over the 16 elements in order of
 * d*d, d = x - fl(e2m1(code) * s * g) (each operation rounded once); ties keep
 * the plain block.  Decoding is unchanged: any NVFP4 consumer reads the result.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_quantize_4over6(const void *x, nvfp4_dtype x_type,
                                   int64_t batch, int64_t rows, int64_t cols,
                                   uint8_t *q, uint8_t *s, float *g,
                                   void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Dense W4A4 GEMM (Model-Optimizer QAD tutorial for Qwen3.6-35B-A3B, section
 * "Why W4A4 rather than W4A16": both operands NVFP4, wide accumulation).
 *
 *   C[m][n] = a_g * b_g * sum_k e2m1(A[m][k]) e4m3(sA[m][k/16])
 *                               * e2m1(B[n][k]) e4m3(sB[n][k/16])
 * i.e. C = A_hat * B_hat^T with A [M x K] (activations) and B [N x K] (weights,
 * one row per output feature), both NVFP4 along K.  Products of decoded
 * operands are exact; accumulation is float32; the global scales are applied
 * once in the epilogue; the result is rounded to c_type.
 * M, N >= 0; K > 0 and a multiple of 16.  c is [M][ldc] of c_type, ldc >= N.
 * a_g, b_g: device floats (read by the kernel; no host synchronization).
 * The fastest path needs K % 256 == 0 and 16-byte aligned q and s; K % 128
 * == 0 with aligned rows takes a vector-load path, other shapes a general
 * path; all give results within the same bound.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_gemm(const uint8_t *a_q, const uint8_t *a_s, const float *a_g,
                        const uint8_t *b_q, const uint8_t *b_s, const float *b_g,
                        int64_t M, int64_t N, int64_t K, void *c,
                        nvfp4_dtype c_type, int64_t ldc, hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8 W8A8 quantize (QAD tutorial for Qwen3.6-35B-A3B, table of quantized
 * tensors: the attention projections of the W4A4 checkpoint stay FP8 W8A8;
 * format-selection guide, section 1: FP8 is W8A8 with per-tensor scaling;
 * two-level scaling page: the family's FP8 is E4M3 with one FP32 scale per
 * tensor that the reader multiplies back in).
 *
 * x       float32 or bfloat16 [rows][ld_x], ld_x >= cols (elements).
 * q       [rows][cols] E4M3FN codes, one byte per element, 16-byte aligned.
 * g       1 float, decode scale: x_hat = e4m3(q) * g.
 *   static_scale == 0: g := amax/448 (1 if all zero), written by the kernel;
 *   static_scale != 0: *g is read as given (finite, >= 2^-100).
 * Encode, float32, round to nearest even: r = 1/g; y = x*r;
 *   q = sign(x) | E4M3(min(|y|, 448))   (saturates; never the NaN code).
 * cols > 0, cols % 16 == 0, rows >= 0, rows * cols / 16 < 2^31.
 * workspace: as for nvfp4_quantize (nvfp4_fp8_quantize_workspace_size bytes,
 * 256-byte aligned, zero-filled before its first use, then reused; not needed
 * with static_scale).  The two quantizers may share one workspace.
 * ---------------------------------------------------------------------- */
size_t nvfp4_fp8_quantize_workspace_size(int64_t rows, int64_t cols);
nvfp4_status nvfp4_fp8_quantize(const void *x, nvfp4_dtype x_type,
                                int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t *q, float *g, int static_scale,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8 W8A8 GEMM (same passages as nvfp4_fp8_quantize).
 *
 *   C[m][n] = a_g * b_g * sum_k e4m3(A[m][k]) * e4m3(B[n][k])
 * A [M x K] activations and B [N x K] weights (one row per output feature),
 * dense row-major E4M3FN bytes, 16-byte aligned.  Products are exact,
 * accumulation is float32, the scales are applied once in the epilogue, the
 * result is rounded to c_type.  M, N >= 0; K > 0, K % 16 == 0; c is
 * [M][ldc] of c_type, ldc >= N.  a_g, b_g: device floats.
 * The fast path needs K % 128 == 0; other K take a general path.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_fp8_gemm(const uint8_t *a_q, const float *a_g,
                            const uint8_t *b_q, const float *b_g,
                            int64_t M, int64_t N, int64_t K, void *c,
                            nvfp4_dtype c_type, int64_t ldc, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MoE routing (two-level scaling page, section "Why only routed experts":
 * each token uses k of E routed experts chosen by a BF16 router).
 *
 * logits  float [T][E] router logits.
 * Top-k: the k largest logits per token, equal logits ordered by lower expert
 * id; slot j holds the j-th largest.  topk_w = softmax over the k selected
 * logits (float32).  Routed rows R = T*k are grouped by expert, then token:
 *   expert_offsets int32 [E+1]  rows of expert e: [offsets[e], offsets[e+1])
 *   src_row        int32 [T*k]  token of routed row r
 *   inv            int32 [T][k] routed row of (token t, slot j)
 *   topk_ids       int32 [T][k], topk_w float [T][k]
 * 1 <= k <= E <= 1024, k <= 32, T >= 0, T*k < 2^31.
 * workspace: nvfp4_moe_route_workspace_size(T, E, k) bytes (clobbered).
 * The order is deterministic (a counting sort, no atomics).
 * ---------------------------------------------------------------------- */
size_t nvfp4_moe_route_workspace_size(int64_t T, int32_t E, int32_t k);
nvfp4_status nvfp4_moe_route(const float *logits, int64_t T, int32_t E,
                             int32_t k, int32_t *topk_ids, float *topk_w,
                             int32_t *expert_offsets, int32_t *src_row,
                             int32_t *inv, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Grouped W4A4 GEMM over expert segments (two-level scaling page, section
 * "Step 1: what NVFP4 touched": the routed experts' fused gate_up_proj and
 * down_proj are the NVFP4 tensors).
 *
 * For every expert e and routed row r in [offsets[e], offsets[e+1]):
 *   acc[r][n] = a_g * w_g[e] * sum_k A_hat[src(r)][k] * W_hat[e][n][k]
 * where src(r) = src_row[r] if src_row != NULL (row gather fused into the
 * operand load) else r.  Every src(r) must lie in [0, a_rows): device-side
 * contents (src_row, expert_offsets) are trusted, not checked.
 * a_q/a_s/a_g  NVFP4 source activations [a_rows][K] (one global scale).
 * expert_offsets  int32 [E+1] on the device, non-decreasing, offsets[0] = 0,
 *              offsets[E] <= R (rows past offsets[E] are not written).
 * R            host upper bound on offsets[E] (sizes the launch).
 * w_q/w_s/w_g  expert weights [E][N][K/2], [E][N][K/16], [E].
 * epilogue     NVFP4_EPI_NONE: c[r][n] = acc (c is [R][N] of c_type);
 *              NVFP4_EPI_SILU_GATE: N = 2I, rows [0, I) of W are the gate and
 *              [I, 2I) the up projection; c[r][i] = SiLU(acc[r][i]) *
 *              acc[r][I+i] with SiLU(z) = z / (1 + exp(-z)), c is [R][I] of
 *              c_type.
 * K > 0, K % 16 == 0; N > 0 (even for SILU_GATE); E >= 1.
 * ---------------------------------------------------------------------- */
typedef enum { NVFP4_EPI_NONE = 0, NVFP4_EPI_SILU_GATE = 1 } nvfp4_epilogue;

nvfp4_status nvfp4_moe_grouped_gemm(
    const uint8_t *a_q, const uint8_t *a_s, const float *a_g, int64_t a_rows,
    const int32_t *src_row, const int32_t *expert_offsets, int32_t E, int64_t R,
    const uint8_t *w_q, const uint8_t *w_s, const float *w_g, int64_t N,
    int64_t K, void *c, nvfp4_dtype c_type, nvfp4_epilogue epilogue,
    hipStream_t stream);

/* ------------------------------------------------------------------------
 * Grouped gate_up GEMM with the SiLU-gate epilogue writing h directly as
 * NVFP4 under a static (calibrated) global scale.  The two-level scaling page
 * calibrates activations with a max over sampled batches (sub-section "The
 * A4 side: dynamic activations"), and its checkpoint audit lists two FP32
 * values per quantized tensor, read here as the weight's global scale and a
 * calibrated activation scale.  With the activation scale known, the down
 * projection's input needs no pass of its own: h = SiLU(gate) * up is
 * quantized in the epilogue of the GEMM that produces it.
 *
 * Same operands and expert segments as nvfp4_moe_grouped_gemm with
 * NVFP4_EPI_SILU_GATE (N = 2I, gate rows [0, I), up rows [I, 2I)); h[r][i] is
 * computed in float32 exactly as that call would return it with c_type
 * NVFP4_F32, then quantized block by block as nvfp4_quantize does with
 * static_global != 0:
 * h_q     uint8 [R][I/2]   codes of h (rows past offsets[E] not written)
 * h_s     uint8 [R][I/16]  E4M3 block scales
 * h_g     device float [1], read: the static global scale of h (a positive
 *         normal float >= 2^-100; values beyond 6*448*h_g saturate)
 * I = N/2 must be a multiple of 16.  This fused path needs K % 256 == 0,
 * a_q, a_s, w_q, w_s 16-byte aligned and h_q 8-byte aligned; other valid
 * requests return NVFP4_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_moe_grouped_gemm_silu_nvfp4(
    const uint8_t *a_q, const uint8_t *a_s, const float *a_g, int64_t a_rows,
    const int32_t *src_row, const int32_t *expert_offsets, int32_t E, int64_t R,
    const uint8_t *w_q, const uint8_t *w_s, const float *w_g, int64_t N,
    int64_t K, uint8_t *h_q, uint8_t *h_s, const float *h_g,
    hipStream_t stream);

/* ------------------------------------------------------------------------
 * Weighted unpermute (combine) of routed-row outputs back to tokens:
 *   out[t][h] = sum_{j=0..k-1} topk_w[t][j] * y[inv[t][j]][h]
 * summed in float32 in slot order, rounded to out_type.
 * y [R][H] of y_type, topk_w float [T][k], inv int32 [T][k], out [T][H].
 * ---------------------------------------------------------------------- */
nvfp4_status nvfp4_moe_combine(const void *y, nvfp4_dtype y_type,
                               const float *topk_w, const int32_t *inv,
                               int64_t T, int32_t k, int64_t H, int64_t R,
                               void *out, nvfp4_dtype out_type,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
