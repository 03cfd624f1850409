// nvfp4_kernels.hpp -- parameter blocks and launchers shared between the
// kernels (*.hip) and the C ABI layer (api.cpp).  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_common.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------- quantize
constexpr uint32_t kMaxPartials = 256;  // amax partials per matrix

// Arrival state of the single-read (resident) quantize kernel; lives at the
// start of the quantize workspace, which must be zero-filled before its first
// use.  Every completed launch leaves it ready for the next one.
constexpr uint32_t kMaxResidentWGs = 1024;
struct ResidentState {
  uint32_t parity;     // which slot array the current launch uses
  uint32_t done;       // workgroups finished in the current launch
  uint32_t fallbacks;  // workgroups whose wait expired (diagnostic; 0 when co-resident)
  // bound on each arrival wait, in polls; 0 (the zero-filled state) means the
  // built-in bound.  The kernels never write it: a caller may set a tiny bound
  // to force the expired-wait path (a test of that path).
  uint32_t spin_limit;
  // slot[p][w] = 0x80000000 | bits(max|x| of workgroup w): arrival flag and
  // value in one word, written and read with relaxed atomics
  uint32_t slot[2][kMaxResidentWGs];
};
constexpr size_t kResidentStateBytes = (sizeof(ResidentState) + 255) / 256 * 256;

struct QuantParams {
  const void *x;      // first element of matrix 0
  int64_t ld;         // row stride of x, elements
  int64_t x_mstride;  // elements between consecutive matrices
  uint32_t rows, nbpr, units;  // nbpr = cols/16, units = rows*nbpr
  FastDiv div_nbpr;
  uint8_t *q;  // [batch][rows][cols/2]
  uint8_t *s;  // [batch][rows][cols/16]
  float *g;    // [batch]
  int64_t q_mstride, s_mstride;  // bytes between matrices
  float *partials;               // [batch][P] workspace
  uint32_t P;                    // partials per matrix
  int static_global;
  int four6;  // block scale by the four-over-six rule (two-pass path)
  // quantize-dequantize: y [rows][ld_y] of the input type receives the decoded
  // values instead of q/s being written (nullptr: plain quantize)
  void *y;
  int64_t ld_y;
  // FP8 W8A8: q [rows][cols] receives one E4M3 code per element, the scale is
  // amax / 448, s is not written
  int fp8;
};

uint32_t quantize_partials_per_matrix(uint64_t units);
// st: resident-kernel state (nullptr: two-pass path only)
hipError_t launch_quantize(QuantParams p, bool bf16, bool vec, uint32_t batch, ResidentState *st,
                           hipStream_t stream);

// -------------------------------------------------------------------- GEMM
struct GemmParams {
  const uint8_t *a_q, *a_s;
  const float *a_g;
  const uint8_t *b_q, *b_s;
  const float *b_g;
  uint32_t M, N, K;
  void *c;
  int64_t ldc;
  // grouped (MoE) mode
  uint32_t a_rows;                // rows of A (the gather's source rows)
  const int32_t *src_row;         // nullable row gather
  const int32_t *expert_offsets;  // [E+1]
  uint32_t E;
  int64_t b_mstride_q, b_mstride_s;  // bytes between expert matrices
  // NVFP4 output of the SiLU-gate epilogue (static global scale h_g)
  uint8_t *h_q, *h_s;
  const float *h_g;
};

enum class OutType { F32, BF16 };
enum class Epilogue { None, SiluGate, SiluGateNvfp4 };

hipError_t launch_gemm(const GemmParams &p, OutType out, hipStream_t stream);
// whether the fused SiLU-gate -> NVFP4 epilogue can run these operands
bool grouped_nvfp4_out_supported(const GemmParams &p);
hipError_t launch_grouped_gemm(const GemmParams &p, uint32_t R, OutType out, Epilogue epi,
                               hipStream_t stream);

// --------------------------------------------------------------- FP8 GEMM
// C [M][N] (ldc) = (a_g b_g) * A B^T with A [M][K] and B [N][K] dense
// row-major E4M3FN bytes (row stride K), K % 16 == 0, 16-byte aligned bases.
struct Fp8GemmParams {
  const uint8_t *a_q;
  const float *a_g;
  const uint8_t *b_q;
  const float *b_g;
  uint32_t M, N, K;
  void *c;
  int64_t ldc;
};

// whether the direct-to-LDS kernel runs these operands (else the plain one)
bool fp8_gemm_dma_ok(const Fp8GemmParams &p);
hipError_t launch_fp8_gemm(const Fp8GemmParams &p, OutType out, hipStream_t stream);

// --------------------------------------------------------------------- MoE
size_t route_workspace_bytes(int64_t T, int32_t E, int32_t k);
hipError_t launch_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *topk_ids,
                        float *topk_w, int32_t *offsets, int32_t *src_row, int32_t *inv,
                        void *workspace, hipStream_t stream);
hipError_t launch_combine(const void *y, bool y_bf16, const float *w, const int32_t *inv, int64_t T,
                          int32_t k, int64_t H, void *out, bool out_bf16, hipStream_t stream);

}  // namespace nvfp4
