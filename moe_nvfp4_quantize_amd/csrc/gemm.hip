// gemm.hip -- W4A4 NVFP4 GEMM and grouped (routed-expert) GEMM on gfx950.
//
// Model-Optimizer QAD tutorial for Qwen3.6-35B-A3B, section "Why W4A4 rather
// than W4A16": both operands are 4-bit NVFP4 so the product can run on the
// matrix units; two-level scaling page (Qwen3.8-Flash-Next-NVFP4), section
// "Core: the W4A4 two-level scaling mechanism": value = e2m1 * e4m3 * fp32.
//
// Design (CDNA4):
//  * CDNA4's block-scaled FP4 MFMA takes one power-of-two (E8M0) scale per 32
//    elements; NVFP4 has an E4M3 scale (3 mantissa bits) per 16.  A product
//    e2m1 * e4m3 has at most 6 significant bits and lies in [2^-10, 2688], so
//    it is exact in f16.  Each operand is therefore decoded in registers to f16
//    (hardware FP4->f16 convert, then one packed multiply by the block scale)
//    and fed to v_mfma_f32_32x32x16_f16 with float32 accumulation.  The global
//    scales are applied once, in the epilogue.
//  * Packed operands stay packed until the last moment: global -> LDS moves
//    0.5625 B per element (codes + scales), so LDS traffic is a quarter of a
//    f16 GEMM's and the tile loads are 128-byte row segments.
//  * K order inside a 256-wide K step is permuted identically for both
//    operands (a GEMM sums over K, so any common order is exact): lane half h of
//    a wave owns packed bytes [64h, 64h + 64) of each row (K elements
//    [128h, 128h + 128)), and MFMA step t consumes its dword t.  One lane then
//    reads its 64 bytes with four 16-byte LDS loads and one 16-byte load of
//    its eight f16 block scales.
//  * LDS rows are padded to 144 bytes so that the 16-byte reads of 8
//    consecutive rows fall in distinct banks.
#include "nvfp4_common.hpp"
#include "nvfp4_format.hpp"
#include "nvfp4_kernels.hpp"

namespace nvfp4 {

namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 256;          // K elements per main-loop step
constexpr int KB = BK / 2;       // packed bytes per row per step
constexpr int SB = BK / 16;      // scales per row per step
constexpr int ROWB = KB + 16;    // padded LDS row of packed codes, bytes
constexpr int SROWH = SB;        // LDS row of f16 scales, halves

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) times one
// f16 block scale -> 8 exact f16 products.
__device__ __forceinline__ half8v decode8(uint32_t w, _Float16 s) {
  const half2v s2 = {s, s};
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  half8v r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// E4M3 scale byte -> f16 (exact: E4M3FN values lie in [2^-9, 448]).
__device__ __forceinline__ _Float16 scale_f16(uint32_t code) {
  return code ? (_Float16)e4m3_value(code & 0x7Fu) : (_Float16)0.0f;
}

template <typename OutT>
__device__ __forceinline__ void store_out(OutT *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float v) {
  *p = (uint16_t)float_to_bf16_bits(v);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// One workgroup computes a BM x BN output tile with (BM/WM) x (BN/WN) waves,
// each owning WM x WN as (WM/32) x (WN/32) MFMA 32x32 tiles.
//  GROUPED: the M tiles walk the expert segments given by expert_offsets; rows
//           may be gathered through src_row; B is the expert's matrix.
//  ALIGNED: K % 256 == 0 and all operand rows 16-byte aligned.
//  SILU:    (GROUPED only, WN == 64) B-tile columns are gate/up pairs and the
//           output is SiLU(gate) * up with N/2 columns.
template <int BM, int BN, int WM, int WN, bool GROUPED, bool ALIGNED, bool SILU, typename OutT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_kernel(GemmParams p) {
  constexpr int NW_N = BN / WN;
  constexpr int NT = (BM / WM) * NW_N * 64;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(!SILU || FN == 2, "SiLU pairing needs two 32-column fragments per wave");

  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[BN * ROWB];
  __shared__ __attribute__((aligned(16))) _Float16 sAs[BM * SROWH];
  __shared__ __attribute__((aligned(16))) _Float16 sBs[BN * SROWH];
  __shared__ int32_t sRow[BM];  // source row of each tile row, -1 past the end
  __shared__ int32_t sInfo[2];  // grouped: expert, first routed row of the tile

  const uint32_t tid = threadIdx.x;
  const uint32_t K = p.K;
  const uint32_t kbytes = K / 2, kscales = K / 16;
  const uint32_t n_out = SILU ? p.N / 2 : p.N;  // output columns
  constexpr uint32_t BN_OUT = SILU ? BN / 2 : BN;
  const uint32_t tiles_n = (n_out + BN_OUT - 1) / BN_OUT;

  // ---- which tile
  uint32_t tile_n, row0, row_end;
  const uint8_t *bq = p.b_q;
  const uint8_t *bs = p.b_s;
  float b_g;
  if (!GROUPED) {
    const uint32_t tiles_m = (p.M + BM - 1) / BM;
    const uint32_t bid = blockIdx.x;
    tile_n = bid / tiles_m;
    row0 = (bid - tile_n * tiles_m) * BM;
    row_end = p.M;
    b_g = *p.b_g;
  } else {
    // tile_mm-th M tile over all experts, each expert contributing ceil(n_e/BM)
    tile_n = blockIdx.x % tiles_n;
    const uint32_t tile_mm = blockIdx.x / tiles_n;
    if (tid == 0) { sInfo[0] = -1; sInfo[1] = 0; }
    __syncthreads();
    // serial scan in chunks of NT experts: thread t owns expert c*NT + t
    uint32_t base = 0;
    for (uint32_t c0 = 0; c0 < p.E; c0 += NT) {
      const uint32_t e = c0 + tid;
      uint32_t cnt = 0, lo = 0;
      if (e < p.E) {
        lo = (uint32_t)p.expert_offsets[e];
        cnt = ((uint32_t)p.expert_offsets[e + 1] - lo + BM - 1) / BM;
      }
      // inclusive prefix over the chunk through LDS
      __shared__ uint32_t scan[NT];
      scan[tid] = cnt;
      __syncthreads();
      for (uint32_t off = 1; off < NT; off <<= 1) {
        uint32_t v = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
      }
      const uint32_t incl = base + scan[tid];
      const uint32_t excl = incl - cnt;
      if (e < p.E && cnt && tile_mm >= excl && tile_mm < incl) {
        sInfo[0] = (int32_t)e;
        sInfo[1] = (int32_t)(lo + (tile_mm - excl) * BM);
      }
      base += scan[NT - 1];
      __syncthreads();
    }
    if (sInfo[0] < 0) return;  // past the last tile (uniform across the workgroup)
    const uint32_t e = (uint32_t)sInfo[0];
    row0 = (uint32_t)sInfo[1];
    row_end = (uint32_t)p.expert_offsets[e + 1];
    bq += (int64_t)e * p.b_mstride_q;
    bs += (int64_t)e * p.b_mstride_s;
    b_g = p.b_g[e];
  }
  const float out_scale = (*p.a_g) * b_g;

  for (uint32_t r = tid; r < BM; r += NT) {
    const uint32_t row = row0 + r;
    int32_t src = -1;
    if (row < row_end) src = (GROUPED && p.src_row) ? p.src_row[row] : (int32_t)row;
    sRow[r] = src;
  }
  // B-tile row rho -> weight row
  auto b_row = [&](uint32_t rho) -> int32_t {
    uint32_t n;
    if (SILU) {
      const uint32_t half = p.N / 2;
      const uint32_t col = tile_n * BN_OUT + (rho / 64) * 32 + (rho % 32);
      if (col >= half) return -1;
      n = ((rho % 64) < 32) ? col : half + col;
    } else {
      n = tile_n * BN + rho;
      if (n >= p.N) return -1;
    }
    return (int32_t)n;
  };
  __syncthreads();

  const uint32_t wave = tid / 64, lane = tid % 64;
  const uint32_t wm = wave / NW_N, wn = wave % NW_N;
  const uint32_t l32 = lane % 32, lh = lane / 32;

  float16v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const uint32_t nsteps = (K + BK - 1) / BK;
  for (uint32_t ks = 0; ks < nsteps; ++ks) {
    const uint32_t kb0 = ks * KB;   // first packed byte of this step
    const uint32_t ksc0 = ks * SB;  // first scale of this step
    __syncthreads();  // previous step's LDS reads are done
    // ---- packed codes: 8 x 16-byte chunks per row
    for (uint32_t c = tid; c < (uint32_t)(BM + BN) * 8; c += NT) {
      const bool isA = c < (uint32_t)BM * 8;
      const uint32_t rho = (isA ? c : c - BM * 8) / 8, ch = c % 8;
      const int32_t src = isA ? sRow[rho] : b_row(rho);
      uint8_t *dst = (isA ? sA : sB) + rho * ROWB + ch * 16;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (src >= 0) {
        const uint8_t *g = (isA ? p.a_q : bq) + (int64_t)src * kbytes + kb0 + ch * 16;
        if (ALIGNED) {
          v = *reinterpret_cast<const u32x4 *>(g);
        } else {
          uint8_t tmp[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) tmp[i] = (kb0 + ch * 16 + i < kbytes) ? g[i] : 0;
          __builtin_memcpy(&v, tmp, 16);
        }
      }
      *reinterpret_cast<u32x4 *>(dst) = v;
    }
    // ---- block scales: 16 per row, converted to f16
    for (uint32_t c = tid; c < (uint32_t)(BM + BN); c += NT) {
      const bool isA = c < (uint32_t)BM;
      const uint32_t rho = isA ? c : c - BM;
      const int32_t src = isA ? sRow[rho] : b_row(rho);
      uint8_t sc[16];
      if (src >= 0) {
        const uint8_t *g = (isA ? p.a_s : bs) + (int64_t)src * kscales + ksc0;
        if (ALIGNED) {
          u32x4 v = *reinterpret_cast<const u32x4 *>(g);
          __builtin_memcpy(sc, &v, 16);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[i] = (ksc0 + i < kscales) ? g[i] : 0;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = 0;
      }
      _Float16 *dst = (isA ? sAs : sBs) + rho * SROWH;
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[i] = scale_f16(sc[i]);
    }
    __syncthreads();

    // ---- fragments: lane (l32, lh) of fragment i reads row (wave row base + 32i + l32)
    u32x4 pa[FM][4], pb[FN][4];
    half8v sa[FM], sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint32_t rho = wm * WM + i * 32 + l32;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(sA + rho * ROWB + lh * 64);
#pragma unroll
      for (int c = 0; c < 4; ++c) pa[i][c] = src[c];
      sa[i] = *reinterpret_cast<const half8v *>(sAs + rho * SROWH + lh * 8);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint32_t rho = wn * WN + j * 32 + l32;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(sB + rho * ROWB + lh * 64);
#pragma unroll
      for (int c = 0; c < 4; ++c) pb[j][c] = src[c];
      sb[j] = *reinterpret_cast<const half8v *>(sBs + rho * SROWH + lh * 8);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      half8v av[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) av[i] = decode8(pa[i][t / 4][t % 4], sa[i][t / 2]);
#pragma unroll
      for (int j = 0; j < FN; ++j) bv[j] = decode8(pb[j][t / 4][t % 4], sb[j][t / 2]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue.  Accumulator register r of lane (l32, lh) in a 32x32 tile
  // holds row 8*(r/4) + 4*lh + (r%4), column l32.
  OutT *C = static_cast<OutT *>(p.c);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t trow = wm * WM + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
      const uint32_t row = row0 + trow;
      if (row >= row_end) continue;
      if (SILU) {
        const uint32_t col = tile_n * BN_OUT + wn * 32 + l32;
        if (col < n_out) {
          const float gt = acc[i][0][r] * out_scale;
          const float up = acc[i][1][r] * out_scale;
          store_out<OutT>(C + (int64_t)row * p.ldc + col, silu(gt) * up);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint32_t col = tile_n * BN + wn * WN + j * 32 + l32;
          if (col < n_out) store_out<OutT>(C + (int64_t)row * p.ldc + col, acc[i][j][r] * out_scale);
        }
      }
    }
  }
}

template <bool GROUPED, bool SILU, typename OutT>
hipError_t launch_cfg(const GemmParams &p, uint32_t grid, bool aligned, hipStream_t stream) {
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  if (aligned)
    gemm_kernel<BM, BN, WM, WN, GROUPED, true, SILU, OutT><<<grid, NT, 0, stream>>>(p);
  else
    gemm_kernel<BM, BN, WM, WN, GROUPED, false, SILU, OutT><<<grid, NT, 0, stream>>>(p);
  return hipGetLastError();
}

bool is_aligned(const GemmParams &p) {
  auto al = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
  return p.K % BK == 0 && al(p.a_q) && al(p.a_s) && al(p.b_q) && al(p.b_s) &&
         p.b_mstride_q % 16 == 0 && p.b_mstride_s % 16 == 0;
}

}  // namespace

hipError_t launch_gemm(const GemmParams &p, OutType out, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const uint32_t grid = ((p.M + 127) / 128) * ((p.N + 127) / 128);
  const bool al = is_aligned(p);
  return out == OutType::BF16 ? launch_cfg<false, false, uint16_t>(p, grid, al, stream)
                              : launch_cfg<false, false, float>(p, grid, al, stream);
}

hipError_t launch_grouped_gemm(const GemmParams &p, uint32_t R, OutType out, Epilogue epi,
                               hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const uint32_t n_out = epi == Epilogue::SiluGate ? p.N / 2 : p.N;
  const uint32_t bn_out = epi == Epilogue::SiluGate ? 64 : 128;
  const uint32_t tiles_n = (n_out + bn_out - 1) / bn_out;
  // sum_e ceil(n_e / BM) <= R / BM + E
  const uint64_t tiles_m = (uint64_t)(R + 127) / 128 + p.E;
  const uint32_t grid = (uint32_t)(tiles_m * tiles_n);
  const bool al = is_aligned(p);
  if (epi == Epilogue::SiluGate)
    return out == OutType::BF16 ? launch_cfg<true, true, uint16_t>(p, grid, al, stream)
                                : launch_cfg<true, true, float>(p, grid, al, stream);
  return out == OutType::BF16 ? launch_cfg<true, false, uint16_t>(p, grid, al, stream)
                              : launch_cfg<true, false, float>(p, grid, al, stream);
}

}  // namespace nvfp4
