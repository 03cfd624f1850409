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
//    and fed to v_mfma_f32_32x32x16_f16 with float32 accumulation; the global
//    scales are applied once, in the epilogue.
//  * Decode of 8 codes (one dword) with block scale s: four hardware FP4->f16
//    converts with unit scale (the convert's own scale operand only applies a
//    power of two, so it cannot carry an E4M3 scale) and four packed f16
//    multiplies by (s, s).  The f16 form of s comes from bits: an E4M3FN byte c
//    shifted left by 7 is an f16 whose value is s * 2^-8 (normal and subnormal
//    alike), and one packed multiply by 256 makes it s.
//  * Packed operands stay packed until the last moment: global -> LDS moves
//    0.5625 B per element (codes + scales), a quarter of an f16 GEMM's LDS
//    traffic.  Two kernels share the decode and the epilogue: gemm_dma_kernel
//    (dense and grouped, K % 256 == 0, aligned operands; described where it is
//    defined) and gemm_kernel (any valid K and alignment, dense and grouped),
//    whose loads go through registers into a double-buffered LDS stage while
//    the current one is multiplied.
//  * Large wave tiles (up to 128 x 128 per wave) amortise each decoded
//    fragment over 4 MFMAs in each direction: the decode work per MFMA falls as
//    1/WM + 1/WN.
//  * K order inside a 128-wide K step is permuted identically for both
//    operands (a GEMM sums over K, so any common order is exact): lane half h of
//    a wave owns packed bytes [32h, 32h + 32) of each row (K elements
//    [64h, 64h + 64), blocks 4h..4h+3), and MFMA step t consumes its dword t.
//  * gemm_kernel pads LDS rows of codes to 80 bytes so the 16-byte reads of 8
//    consecutive rows fall in distinct banks; gemm_dma_kernel swizzles them.
//  * The epilogue stages each wave's 32-row slab through LDS so that global
//    stores are 16 bytes per lane along a row.
//  * Dense tiles are ordered XCD-aware: workgroup w runs on XCD w % 8, so each
//    XCD is given a contiguous range of tiles, swept 8 tile-rows at a time so
//    that concurrently running workgroups share A and B tiles in that XCD's L2.
#include "nvfp4_common.hpp"
#include "nvfp4_format.hpp"
#include "nvfp4_kernels.hpp"

namespace nvfp4 {

namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr int BK = 128;        // K elements per stage
constexpr int KB = BK / 2;     // packed bytes per row per stage
constexpr int SBY = BK / 16;   // scale bytes per row per stage
constexpr int ROWB = KB + 16;  // padded LDS row of codes, bytes

template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN, NT = NW * 64;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int CHA = BM * 4 / NT, CHB = BN * 4 / NT;  // 16-byte code chunks per thread
  static constexpr int OFF_B = BM * ROWB;
  static constexpr int OFF_SA = OFF_B + BN * ROWB;
  static constexpr int OFF_SB = OFF_SA + BM * SBY;
  static constexpr int STAGE = OFF_SB + BN * SBY;
  static_assert(BM * 4 % NT == 0 && BN * 4 % NT == 0, "code chunks must split evenly");
};

// two E4M3FN scale bytes (bits 7..0 and 23..16 of w) -> f16 pair of the
// scales divided by 256 (exact): the bytes moved up by 7 bits are the f16
// encodings of s / 2^8 (f16 exponent bias 15 against E4M3's 7; E4M3
// subnormals land on f16 subnormals); decode8 applies the factor 2^8 in its
// code conversion instead of a multiply here
__device__ __forceinline__ half2v scale_pair(uint32_t w) {
  return __builtin_bit_cast(half2v, (w & 0x00FF00FFu) << 7);
}

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) times the
// block scale s, given as s / 256 (scale_pair) -> 8 exact f16 products: the
// conversion multiplies the codes by its power-of-two scale operand exactly
// (codes x 256 <= 1536), and code x s needs at most 6 significant bits
// between 2^-10 and 2688, well inside f16
__device__ __forceinline__ half8v decode8(uint32_t w, _Float16 s) {
  const half2v s2 = {s, s};
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s2;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s2;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s2;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s2;
  return (half8v){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// SiLU(z) = z / (1 + e^-z), with e^-z = 2^(-z log2 e) from the hardware base-2
// exponential and the quotient from the hardware reciprocal (about 1 ulp each;
// below z = -88.7 the power overflows to inf and the result is a signed zero).  The epilogue
// evaluates one per output: the IEEE division and the range-reduced exp were
// long dependent chains there.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

template <typename OutT>
__device__ __forceinline__ OutT to_out(float v);
template <>
__device__ __forceinline__ float to_out<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t to_out<uint16_t>(float v) { return (uint16_t)float_to_bf16_bits(v); }

// One workgroup computes a BM x BN tile of acc with NWM x NWN waves, each
// owning WM x WN as FM x FN MFMA 32x32 tiles.
//  GROUPED: M tiles walk the expert segments given by expert_offsets; rows may
//           be gathered through src_row; B is the expert's matrix.
//  ALIGNED: K % 128 == 0 and q/s bases 16/8-byte aligned: vector loads.
//  SILU:    (GROUPED only) in every wave the first FN/2 fragments hold gate
//           columns and the last FN/2 the matching up columns; the output is
//           SiLU(gate) * up with N/2 columns.
//  VSTORE:  output rows are 16-byte aligned: 16-byte stores.
template <int BM, int BN, int WM, int WN, bool GROUPED, bool ALIGNED, bool SILU, bool VSTORE,
          typename OutT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void gemm_kernel(GemmParams p) {
  using TL = Tile<BM, BN, WM, WN>;
  constexpr int NT = TL::NT, FM = TL::FM, FN = TL::FN, NWN = TL::NWN;
  constexpr int HALF = FN / 2;
  static_assert(!SILU || FN % 2 == 0, "SiLU pairing needs an even number of column fragments");
  constexpr uint32_t BN_OUT = SILU ? BN / 2 : BN;
  constexpr int WN_OUT = SILU ? WN / 2 : WN;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::STAGE];
  __shared__ int32_t sRow[BM];  // source row of each tile row, -1 past the end
  __shared__ int32_t sInfo[2];

  const uint32_t tid = threadIdx.x;
  const uint32_t K = p.K;
  const uint32_t kbytes = K / 2, kscales = K / 16;
  const uint32_t n_out = SILU ? p.N / 2 : p.N;
  const uint32_t tiles_n = (n_out + BN_OUT - 1) / BN_OUT;

  // ---------------------------------------------------------------- tile
  uint32_t tile_n, row0, row_end;
  const uint8_t *bq = p.b_q;
  const uint8_t *bs = p.b_s;
  float b_g;
  if (!GROUPED) {
    const uint32_t tiles_m = (p.M + BM - 1) / BM;
    uint32_t tm;
    dense_tile(blockIdx.x, tiles_m, tiles_n, &tm, &tile_n);
    row0 = tm * BM;
    row_end = p.M;
    b_g = *p.b_g;
  } else {
    // tile_mm-th M tile over all experts, expert e contributing ceil(n_e / BM)
    tile_n = blockIdx.x % tiles_n;
    const uint32_t tile_mm = blockIdx.x / tiles_n;
    __shared__ uint32_t scan[NT];
    if (tid == 0) sInfo[0] = -1;
    uint32_t base = 0;
    for (uint32_t c0 = 0; c0 < p.E; c0 += NT) {
      const uint32_t e = c0 + tid;
      uint32_t cnt = 0, lo = 0;
      if (e < p.E) {
        lo = (uint32_t)p.expert_offsets[e];
        cnt = ((uint32_t)p.expert_offsets[e + 1] - lo + BM - 1) / BM;
      }
      scan[tid] = cnt;
      __syncthreads();
      for (uint32_t off = 1; off < NT; off <<= 1) {
        const uint32_t v = tid >= off ? scan[tid - off] : 0;
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
    if (sInfo[0] < 0) return;  // past the last tile: the whole workgroup leaves
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
  // B-tile row rho -> weight row (or -1 past N)
  auto b_row = [&](uint32_t rho) -> int32_t {
    if (SILU) {
      const uint32_t half = p.N / 2;
      const uint32_t wn = rho / WN, j = (rho % WN) / 32, c = rho % 32;
      const uint32_t col = tile_n * BN_OUT + wn * (WN / 2) + (j % HALF) * 32 + c;
      if (col >= half) return -1;
      return (int32_t)(j < (uint32_t)HALF ? col : half + col);
    }
    const uint32_t n = tile_n * BN + rho;
    return n < p.N ? (int32_t)n : -1;
  };
  __syncthreads();

  // per-thread source rows of the code chunks it loads (fixed over K)
  int32_t srcA[TL::CHA], srcB[TL::CHB];
#pragma unroll
  for (int i = 0; i < TL::CHA; ++i) srcA[i] = sRow[(tid + i * NT) / 4];
#pragma unroll
  for (int i = 0; i < TL::CHB; ++i) srcB[i] = b_row((tid + i * NT) / 4);
  constexpr int SCH = (BM + BN + NT - 1) / NT;  // scale rows per thread
  int32_t srcS[SCH];
#pragma unroll
  for (int i = 0; i < SCH; ++i) {
    const uint32_t c = tid + i * NT;
    srcS[i] = c < (uint32_t)BM ? sRow[c] : (c < (uint32_t)(BM + BN) ? b_row(c - BM) : -1);
  }

  u32x4 ra[TL::CHA], rb[TL::CHB];
  u32x2 rs[SCH];
  auto load_global = [&](uint32_t ks) {
    const uint32_t kb0 = ks * KB, ksc0 = ks * SBY;
#pragma unroll
    for (int i = 0; i < TL::CHA + TL::CHB; ++i) {
      const bool isA = i < TL::CHA;
      const uint32_t c = tid + (isA ? i : i - TL::CHA) * NT;
      const int32_t src = isA ? srcA[i] : srcB[i - TL::CHA];
      const uint32_t off = kb0 + (c % 4) * 16;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (src >= 0) {
        const uint8_t *g = (isA ? p.a_q : bq) + (int64_t)src * kbytes + off;
        if (ALIGNED) {
          v = *reinterpret_cast<const u32x4 *>(g);
        } else {
          uint8_t tmp[16];
#pragma unroll
          for (int b = 0; b < 16; ++b) tmp[b] = (off + b < kbytes) ? g[b] : 0;
          __builtin_memcpy(&v, tmp, 16);
        }
      }
      if (isA) ra[i] = v; else rb[i - TL::CHA] = v;
    }
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const uint32_t c = tid + i * NT;
      u32x2 v = {0u, 0u};
      if (srcS[i] >= 0) {
        const uint8_t *g = (c < (uint32_t)BM ? p.a_s : bs) + (int64_t)srcS[i] * kscales + ksc0;
        if (ALIGNED) {
          v = *reinterpret_cast<const u32x2 *>(g);
        } else {
          uint8_t tmp[8];
#pragma unroll
          for (int b = 0; b < 8; ++b) tmp[b] = (ksc0 + b < kscales) ? g[b] : 0;
          __builtin_memcpy(&v, tmp, 8);
        }
      }
      rs[i] = v;
    }
  };
  auto store_lds = [&](uint32_t buf) {
    uint8_t *st = smem + buf * TL::STAGE;
#pragma unroll
    for (int i = 0; i < TL::CHA; ++i) {
      const uint32_t c = tid + i * NT;
      *reinterpret_cast<u32x4 *>(st + (c / 4) * ROWB + (c % 4) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < TL::CHB; ++i) {
      const uint32_t c = tid + i * NT;
      *reinterpret_cast<u32x4 *>(st + TL::OFF_B + (c / 4) * ROWB + (c % 4) * 16) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const uint32_t c = tid + i * NT;
      if (c < (uint32_t)(BM + BN)) *reinterpret_cast<u32x2 *>(st + TL::OFF_SA + c * SBY) = rs[i];
    }
  };

  const uint32_t wave = tid / 64, lane = tid % 64;
  const uint32_t wm = wave / NWN, wn = wave % NWN;
  const uint32_t l32 = lane % 32, lh = lane / 32;

  float16v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](uint32_t buf) {
    const uint8_t *st = smem + buf * TL::STAGE;
    u32x4 pa[FM][2], pb[FN][2];
    half2v sa[FM][2], sb[FN][2];  // (scale of block 2m, of block 2m+1) for m = 0, 1
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint32_t rho = wm * WM + i * 32 + l32;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(st + rho * ROWB + lh * 32);
      pa[i][0] = src[0];
      pa[i][1] = src[1];
      const uint32_t w = *reinterpret_cast<const uint32_t *>(st + TL::OFF_SA + rho * SBY + lh * 4);
      sa[i][0] = scale_pair(w);       // blocks 0, 2 of the lane's four
      sa[i][1] = scale_pair(w >> 8);  // blocks 1, 3
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint32_t rho = wn * WN + j * 32 + l32;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(st + TL::OFF_B + rho * ROWB + lh * 32);
      pb[j][0] = src[0];
      pb[j][1] = src[1];
      const uint32_t w = *reinterpret_cast<const uint32_t *>(st + TL::OFF_SB + rho * SBY + lh * 4);
      sb[j][0] = scale_pair(w);
      sb[j][1] = scale_pair(w >> 8);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      // dword t covers block t/2 of the lane's four: scale_pair slot (t/2)%2, lane (t/2)/2
      const int blk = t / 2;
      half8v av[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) av[i] = decode8(pa[i][t / 4][t % 4], sa[i][blk % 2][blk / 2]);
#pragma unroll
      for (int j = 0; j < FN; ++j) bv[j] = decode8(pb[j][t / 4][t % 4], sb[j][blk % 2][blk / 2]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };

  // ---------------------------------------------------------------- K loop
  const uint32_t nsteps = (K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  if (nsteps > 1) load_global(1);
  for (uint32_t ks = 0; ks < nsteps; ++ks) {
    compute(ks & 1);
    if (ks + 1 < nsteps) store_lds((ks + 1) & 1);
    __syncthreads();
    if (ks + 2 < nsteps) load_global(ks + 2);
  }

  // ---------------------------------------------------------------- epilogue
  // Each wave stages one 32-row slab (its fragment row i) at a time in its own
  // LDS region, then writes it out row by row.  Accumulator register r of lane
  // (l32, lh) in a 32x32 tile holds row 8*(r/4) + 4*lh + (r%4), column l32.
  constexpr int ROW_ELEMS = WN_OUT;
  constexpr int ROW_BYTES = ROW_ELEMS * (int)sizeof(OutT) + 16;  // +16: bank spread
  static_assert(TL::NW * 32 * ROW_BYTES <= 2 * TL::STAGE, "epilogue staging must fit");
  OutT *C = static_cast<OutT *>(p.c);
  uint8_t *slab = smem + wave * 32 * ROW_BYTES;
  const uint32_t col0 = tile_n * BN_OUT + wn * WN_OUT;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t tr = 8 * (r / 4) + 4 * lh + (r % 4);
      OutT *dst = reinterpret_cast<OutT *>(slab + tr * ROW_BYTES);
      if (SILU) {
#pragma unroll
        for (int j = 0; j < HALF; ++j)
          dst[j * 32 + l32] =
              to_out<OutT>(silu(acc[i][j][r] * out_scale) * (acc[i][j + HALF][r] * out_scale));
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) dst[j * 32 + l32] = to_out<OutT>(acc[i][j][r] * out_scale);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    // 32 rows x ROW_ELEMS outputs, 16 bytes (VEC elements) per lane-chunk
    constexpr int VEC = 16 / (int)sizeof(OutT);
    constexpr int CPR = ROW_ELEMS / VEC;  // chunks per row
    const uint32_t rbase = row0 + wm * WM + i * 32;
    for (int c = lane; c < 32 * CPR; c += 64) {
      const uint32_t tr = c / CPR, cc = c % CPR;
      const uint32_t row = rbase + tr;
      const uint32_t col = col0 + cc * VEC;
      if (row >= row_end) continue;
      const uint8_t *srcp = slab + tr * ROW_BYTES + cc * 16;
      OutT *g = C + (int64_t)row * p.ldc + col;
      if (VSTORE && col + VEC <= n_out) {
        *reinterpret_cast<u32x4 *>(g) = *reinterpret_cast<const u32x4 *>(srcp);
      } else {
        const OutT *sv = reinterpret_cast<const OutT *>(srcp);
        for (int e = 0; e < VEC; ++e)
          if (col + e < n_out) g[e] = sv[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}


// ====================================================================
// Main kernel (dense and grouped) for K % 256 == 0 and aligned operands:
// global -> LDS without registers, software-pipelined decode.
// ====================================================================

// Grouped launches without the SiLU gate (down projections) and with short K
// loops walk two N tiles of one M tile per workgroup (the second tile's first K
// steps are fetched during the first's last ones; both use the same gathered
// rows) when whole scale chunks tile K and the N tiles pair up.  Measured on
// the 512-expert layer: down (K = 1024) -6%; gate_up (K = 4096) +4% (half as
// many workgroups to balance over the CUs, and a prologue that 32 K steps
// already hide), and the walk's code alone cost the gate_up kernel 3%, so it is
// compiled into the kernels without the gate only.  Not with 256-row tiles: the
// walk's state does not fit their registers.
__host__ __device__ inline bool grouped_walk(int bm, bool silu, uint32_t K, uint32_t n_out, uint32_t bn_out) {
  return bm != 256 && !silu && K % 1024 == 0 && K <= 2048 && n_out % bn_out == 0 &&
         (n_out / bn_out) % 2 == 0;
}

// BM x BN output tile (BM = 128, 192 or 256; BN = 256, or 320 for dense
// products of at most 128 rows), four waves: 2 x 2 of BM/2 x BN/2 (BM/64 x
// BN/64 MFMA tiles each), or, for 128 x 256 tiles and grouped 192-row tiles,
// 1 x 4 of BM x 64 (BM/32 x 2 MFMA tiles each).  The MFMAs take the weight
// fragment first, so an accumulator holds runs of output columns of one row
// (the epilogue below).
//  * Codes and scales go from global memory straight into LDS (64 lanes x 16
//    bytes into 1 KB of consecutive LDS per transfer: buffer_load_dwordx4 ...
//    lds for the codes of dense tiles, whose buffer range ends at the
//    matrix's last row, global_load_lds_dwordx4 otherwise), so no registers
//    hold staged data and no LDS store instructions run.
//  * Codes: three stages of one K step (128 elements: 64 bytes per row),
//    fetched two steps ahead (four stages, three steps ahead, for 128 x 256
//    tiles).  Scales: two chunks of eight K steps (64 bytes per
//    row), so that a transfer reads 64 contiguous bytes of a row instead of 8;
//    the next chunk is fetched during the first four steps of the current one.
//  * Each step issues the same number of transfers ((BM + BN)/64 code, one A
//    and one or two B scale transfers; extra ones reload data that is not read
//    any more, or rewrite identical bytes), so one wait count serves
//    every step: at the mid-step barrier only the step's own transfers may be
//    in flight.  The transfers are spread over the step's MFMAs so that the
//    memory pipeline never backs up the wave's in-order issue.
//  * Fragments are double buffered in registers by half step (16-byte piece):
//    the second half of step k is read at the start of step k, the first half
//    of step k + 1 right after the mid-step barrier.
//  * Decode is software pipelined: while the MFMAs of sub-step t run (16 for
//    256-row tiles), the operands of sub-step t + 1 are decoded (one MFMA, then
//    a few VALU instructions, in turn).
// The fragments a wave multiplies in a tile: F of A (row groups) and FB of B.
template <int F_, int FB_>
struct Frags {
  static constexpr int F = F_, FB = FB_;
};

template <int BM, bool GROUPED, bool SILU, bool VSTORE, typename OutT, bool QOUT = false, int NWM = 2,
          int BN = 256>
__global__ __launch_bounds__(256, 1) void gemm_dma_kernel(GemmParams p) {
  // NWM x NWN waves: 2 x 2 (waves of BM/2 x BN/2) or 1 x 4 (BM x BN/4)
  constexpr int NWN = 4 / NWM;
  constexpr int WM = BM / NWM, WN = BN / NWN, FM = WM / 32, FN = WN / 32, HALF = FN / 2;
  static_assert(BM == 128 || BM == 192 || BM == 256, "tile height");
  static_assert(BN == 256 || (BN == 320 && BM == 128 && NWM == 2 && !GROUPED),
                "320-column tiles: dense products of at most 128 rows, 2 x 2 waves of 64 x 160");
  static_assert(NWM == 1 || NWM == 2, "wave grid");
  static_assert(FM <= 8, "at most eight A fragments per wave");
  static_assert(!QOUT || NWM == 2, "the NVFP4 epilogue quantizes 64-column wave slabs");
  static_assert(!SILU || GROUPED, "the SiLU epilogue is a grouped-GEMM epilogue");
  static_assert(!QOUT || (SILU && sizeof(OutT) == 4), "NVFP4 output: SiLU-gate epilogue, f32 staging");
  // transfers (64 lanes x 16 bytes) per operand: per code stage, and per scale chunk
  constexpr int TA = BM / 64, TB = BN / 64, TN = TA + TB;
  // scale transfers per K step: one of A, NSB of B (a chunk's TB transfers of
  // B spread over its first four steps)
  constexpr int NSB = (TB + 3) / 4, NSC = 1 + NSB;
  // code stages: [A BM rows x 64 B][B BN rows x 64 B], fetched AHEAD steps
  // ahead: four stages for 128 x 256 tiles (skinny products stream their
  // weights from HBM, so the fetch has to run further ahead; 144 KB of LDS),
  // three otherwise (a fourth would not fit)
  constexpr int CODE_B = BM * 64, CODE_STAGE = (BM + BN) * 64, NSTAGE = (BM == 128 && BN == 256) ? 4 : 3;
  constexpr int AHEAD = NSTAGE - 1;
  // scale chunks: the scales of SC_STEPS K steps, [A BM rows x 64 B][B ...], two of them
  constexpr int SC_STEPS = 8, SC_B = BM * 64, SC_CHUNK = (BM + BN) * 64;
  constexpr int OFF_SC = NSTAGE * CODE_STAGE;
  constexpr uint32_t BN_OUT = SILU ? BN / 2 : BN;
  constexpr int WN_OUT = SILU ? WN / 2 : WN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[OFF_SC + 2 * SC_CHUNK];
  // set-up tables, in LDS that the transfers overwrite only after the set-up:
  // the grouped tile search's prefix sums, its result, the tile's source rows
  uint32_t *scan = reinterpret_cast<uint32_t *>(smem);
  int32_t *sInfo = reinterpret_cast<int32_t *>(smem + 1024);
  int32_t *sRow = reinterpret_cast<int32_t *>(smem + 2048);  // -1 past the end

  const uint32_t tid = threadIdx.x;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const uint32_t K = p.K, kbytes = K / 2, kscales = K / 16;
  const uint32_t n_out = SILU ? p.N / 2 : p.N;
  const uint32_t tiles_n = (n_out + BN_OUT - 1) / BN_OUT;
  const uint32_t nsteps = K / 128, cpt = (nsteps + SC_STEPS - 1) / SC_STEPS;
  const bool gwalk = GROUPED && !SILU && BM != 256 && grouped_walk(BM, SILU, K, n_out, BN_OUT);

  // ---------------------------------------------------------------- tiles
  // Dense: workgroup b computes work items b, b + G, b + 2G, ... (G =
  // gridDim.x; when it exceeds one item per workgroup it is a multiple of 8,
  // so they all map to the XCD of b; the host launches more than one item per
  // workgroup only when K % 1024 == 0).  An item is a whole tile, except when
  // the tiles left for the last round fill at most half of it: each of those
  // is then split into its two halves of BM / 2 rows, which run on two
  // workgroups of the same XCD (w and w + 8), so that round takes about half
  // as long.  Grouped: one tile.
  uint32_t my_tiles, row0, row_end, tile_n;
  const uint8_t *bq = p.b_q, *bs = p.b_s;
  float b_g;
  uint32_t tiles_m = 0, full = 0, rem = 0;
  bool split = false;
  uint32_t g_row0 = 0, g_row_end = 0, g_tn0 = 0;  // grouped: the walk's M tile and first N tile
  auto origin = [&](uint32_t i, uint32_t *r0, uint32_t *re, uint32_t *tn) {
    if constexpr (GROUPED) {
      *r0 = g_row0;
      *re = g_row_end;
      *tn = g_tn0 + i;
      return;
    }
    uint32_t tm;
    const uint32_t w = blockIdx.x + i * gridDim.x;
    if (split && w >= full * gridDim.x) {
      // half j of the last round: halves of tile k on workgroups of one XCD
      const uint32_t j = w - full * gridDim.x, nb = (2 * rem) / 16;
      uint32_t k, half;
      if (j < nb * 16) {
        k = (j / 16) * 8 + j % 8;
        half = (j / 8) % 2;
      } else {
        k = nb * 8 + (j - nb * 16) / 2;
        half = (j - nb * 16) % 2;
      }
      dense_tile(full * gridDim.x + k, tiles_m, tiles_n, &tm, tn);
      *r0 = tm * BM + half * (BM / 2);
      *re = min(*r0 + BM / 2, p.M);
    } else {
      dense_tile(w, tiles_m, tiles_n, &tm, tn);
      *r0 = tm * BM;
      *re = p.M;
    }
  };
  if (!GROUPED) {
    tiles_m = (p.M + BM - 1) / BM;
    const uint32_t ntiles = tiles_m * tiles_n;
    full = ntiles / gridDim.x;
    rem = ntiles % gridDim.x;
    split = rem != 0 && 2 * rem <= gridDim.x && p.M > BM / 2;
    const uint32_t items = split ? full * gridDim.x + 2 * rem : ntiles;
    if (blockIdx.x >= items) return;
    my_tiles = (items - 1 - blockIdx.x) / gridDim.x + 1;
    origin(0, &row0, &row_end, &tile_n);
    b_g = *p.b_g;
  } else {
    // tile_mm-th M tile over all experts, expert e contributing ceil(n_e / BM);
    // a work item is one N tile of an M tile (with the walk: N tiles 2j and
    // 2j + 1, one after the other).  Workgroup b runs on XCD b % 8, and XCD x
    // takes the contiguous run of items [x n / 8, (x + 1) n / 8) of the n real
    // items in M-major order (n is known once the scan below has counted the
    // experts' tiles; the grid covers an upper bound): every XCD gets the same
    // share of the real work, the N tiles of an M tile run back to back on one
    // XCD (its gathered rows fetched into that L2 once), and so do the M tiles of
    // one expert, whose weight panels its L2 then serves to both.
    const uint32_t tpw = gwalk ? 2u : 1u, npairs = tiles_n / tpw;
    my_tiles = tpw;
    if (tid == 0) sInfo[0] = -1;
    // Exclusive prefix over experts of ceil(n_e / BM) in one pass: thread t owns
    // experts [t * per, t * per + per); a scan of the threads' sums inside each
    // wave, then the four waves' totals through LDS.
    const uint32_t per = (p.E + 255) / 256, e_lo = tid * per, e_hi = min(e_lo + per, p.E);
    uint32_t own = 0;
    for (uint32_t e = e_lo; e < e_hi; ++e)
      own += ((uint32_t)p.expert_offsets[e + 1] - (uint32_t)p.expert_offsets[e] + BM - 1) / BM;
    uint32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off, 64);
      if (lane >= (uint32_t)off) incl += v;
    }
    if (lane == 63) scan[wave] = incl;
    __syncthreads();
    uint32_t first = incl - own;  // M tiles before this thread's first expert
    for (uint32_t w = 0; w < wave; ++w) first += scan[w];
    const uint32_t items = (scan[0] + scan[1] + scan[2] + scan[3]) * npairs;
    const uint32_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    const uint32_t it0 = (uint32_t)((uint64_t)xcd * items / 8), it1 = (uint32_t)((uint64_t)(xcd + 1) * items / 8);
    uint32_t tile_mm = 0xFFFFFFFFu;  // past the real items: no thread matches
    tile_n = 0;
    if (local < it1 - it0) {
      tile_mm = (it0 + local) / npairs;
      tile_n = ((it0 + local) % npairs) * tpw;
    }
    if (tile_mm >= first && tile_mm < first + own) {
      for (uint32_t e = e_lo; e < e_hi; ++e) {
        const uint32_t lo = (uint32_t)p.expert_offsets[e];
        const uint32_t cnt = ((uint32_t)p.expert_offsets[e + 1] - lo + BM - 1) / BM;
        if (tile_mm < first + cnt) {
          sInfo[0] = (int32_t)e;
          sInfo[1] = (int32_t)(lo + (tile_mm - first) * BM);
          break;
        }
        first += cnt;
      }
    }
    __syncthreads();
    if (sInfo[0] < 0) return;  // past the last tile: the whole workgroup leaves
    const uint32_t e = (uint32_t)sInfo[0];
    row0 = (uint32_t)sInfo[1];
    row_end = (uint32_t)p.expert_offsets[e + 1];
    g_row0 = row0;
    g_row_end = row_end;
    g_tn0 = tile_n;
    bq += (int64_t)e * p.b_mstride_q;
    bs += (int64_t)e * p.b_mstride_s;
    b_g = p.b_g[e];
    for (uint32_t r = tid; r < BM; r += 256) {
      const uint32_t row = row0 + r;
      int32_t src = -1;
      if (row < row_end) src = p.src_row ? p.src_row[row] : (int32_t)row;
      sRow[r] = src;
    }
  }
  const float out_scale = (*p.a_g) * b_g;
  // static global scale of an NVFP4 output (QOUT)
  const float h_g = QOUT ? *p.h_g : 1.0f;
  const float h_six_g = 6.0f * h_g, h_inv_six_g = 1.0f / h_six_g;
  // B-tile row rho -> weight row (or -1 past N).  With SILU, in every wave the
  // first FN/2 fragments hold gate columns and the last FN/2 the matching up
  // columns (weight rows n and N/2 + n).
  // (a grouped walk takes the rows of N tile 0 and adds each tile's first row,
  // b_base below: every tile of such a walk is whole)
  auto b_row = [&](uint32_t rho) -> int32_t {
    const uint32_t tn = gwalk ? 0u : tile_n;
    if (SILU) {
      const uint32_t half = p.N / 2;
      const uint32_t wn = rho / WN, j = (rho % WN) / 32, c = rho % 32;
      const uint32_t col = tn * BN_OUT + wn * (WN / 2) + (j % HALF) * 32 + c;
      if (col >= half) return -1;
      return (int32_t)(j < (uint32_t)HALF ? col : half + col);
    }
    const uint32_t n = tn * BN + rho;
    return n < p.N ? (int32_t)n : -1;
  };
  __syncthreads();

  // Global -> LDS transfers.  One transfer moves 64 lanes x 16 bytes into 1 KB
  // of consecutive LDS: transfer j of an operand covers slots s = j * 256 + tid,
  // i.e. tile row s / 4, physical 16-byte piece s % 4, which holds logical
  // piece (s % 4) ^ swz(row) = pc for every j.  Dense tiles keep the lane
  // part l of a byte offset (row inside the tile): their codes load through a
  // buffer resource based at the tile's first row, whose range check drops
  // rows past the end of the matrix, and their scales at min(l + base, last),
  // clamped to the last row (rows past the end are never stored); grouped
  // tiles hold the full offset of the gathered row (base 0, no clamp).
  // Offsets fit 32 bits (checked by the host).
  const uint32_t pc = (tid % 4) ^ swz(tid / 4);
  // (vectors, not arrays: an index known only at run time becomes selects)
  typedef std::conditional_t<(TB > 4), u32x8, u32x4> BOffsets;
  u32x4 la = {0, 0, 0, 0}, lsa = {0, 0, 0, 0};
  BOffsets lb, lsb;
  uint32_t last_sa, last_sb;
  if (!GROUPED) {
#pragma unroll
    for (int j = 0; j < TA; ++j) {
      la[j] = (j * 64 + tid / 4) * kbytes + pc * 16;
      lsa[j] = (j * 64 + tid / 4) * kscales + pc * 16;
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      lb[j] = (j * 64 + tid / 4) * kbytes + pc * 16;
      lsb[j] = (j * 64 + tid / 4) * kscales + pc * 16;
    }
    last_sa = (p.M - 1) * kscales + pc * 16;
    last_sb = (p.N - 1) * kscales + pc * 16;
  } else {
    const int32_t a_fallback = sRow[0];  // the tile's first row always exists
#pragma unroll
    for (int j = 0; j < TA; ++j) {
      const int32_t src = sRow[j * 64 + tid / 4];
      const uint32_t ra = (uint32_t)(src >= 0 ? src : a_fallback);
      la[j] = ra * kbytes + pc * 16;
      lsa[j] = ra * kscales + pc * 16;
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int32_t w = b_row(j * 64 + tid / 4);
      const uint32_t rb = (uint32_t)(w >= 0 ? w : 0);
      lb[j] = rb * kbytes + pc * 16;
      lsb[j] = rb * kscales + pc * 16;
    }
    last_sa = last_sb = 0xFFFFFFFFu;
  }
  __syncthreads();  // every wave is done with the set-up tables
  // first A row and first B row of a tile as used in the offsets (grouped: A
  // rows are gathered in full, B rows are whole unless the workgroup walks)
  auto a_base = [&](uint32_t r0) { return GROUPED ? 0u : r0; };
  auto b_base = [&](uint32_t tn) { return GROUPED ? (gwalk ? tn * BN_OUT : 0u) : tn * BN; };
  // Dense tiles load through buffer resources that start at the tile's first
  // row and end at the matrix's last byte: a lane whose row lies past the end
  // is out of range and reads nothing from memory (those rows are never
  // stored), so the lane offsets are rows inside the tile, need no clamp, and
  // the K offset is a scalar.  Grouped tiles keep the full per-lane offsets of
  // their gathered rows.
  typedef __amdgpu_buffer_rsrc_t Rsrc;
  auto rsrc = [&](const uint8_t *base, uint32_t bytes) -> Rsrc {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
  };
  // the code stream's fetch tile (dense: its resources; grouped: its first
  // rows as used in the offsets) and the scale stream's target tile (its first
  // rows as used in the offsets)
  Rsrc rA = rsrc(p.a_q, 0), rB = rA;
  uint32_t f_ar = 0, f_bc = 0, s_ar = 0, s_bc = 0;
  auto set_fetch = [&](uint32_t r0, uint32_t tn) {
    if constexpr (!GROUPED) {
      // (the second half of a split tile can start past the last row: empty)
      rA = rsrc(p.a_q + (size_t)r0 * kbytes, p.M > r0 ? (p.M - r0) * kbytes : 0u);
      rB = rsrc(bq + (size_t)tn * BN * kbytes, p.N > tn * BN ? (p.N - tn * BN) * kbytes : 0u);
    } else {
      f_ar = a_base(r0);
      f_bc = b_base(tn);
    }
  };
  auto set_scale_target = [&](uint32_t r0, uint32_t tn) {
    s_ar = a_base(r0);
    s_bc = b_base(tn);
  };
  // code transfer q (0 .. TN - 1; A first) of K step ks of the fetch tile,
  // into the stage at byte offset st
  auto issue_code = [&](uint32_t st, uint32_t ks, int q) {
    lds_void *dst = (lds_void *)(smem + st + (q < TA ? q * 4096 : CODE_B + (q - TA) * 4096) + wave * 1024);
    if constexpr (!GROUPED) {
      // (plain int operands: vector elements passed straight to the builtin
      // make the host compilation drop the kernel's launch stub)
      if (q < TA) __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, dst, 16, (int)(uint32_t)la[q], (int)(ks * 64), 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, dst, 16, (int)(uint32_t)lb[q - TA], (int)(ks * 64), 0, 0);
    } else {
      if (q < TA) __builtin_amdgcn_global_load_lds((glb_void *)(p.a_q + ks * 64 + la[q] + f_ar * kbytes), dst, 16, 0, 0);
      else __builtin_amdgcn_global_load_lds((glb_void *)(bq + ks * 64 + lb[q - TA] + f_bc * kbytes), dst, 16, 0, 0);
    }
  };
  // Scale transfers of part q (0..3) of chunk s_c of the target tile, into the
  // buffer at s_buf: A transfer q % TA and B transfers q, q + 4, ... (the last
  // one repeated past TB; q is not known at compile time).  A piece past the
  // end of the row reloads the chunk's first piece instead.  Dense tiles:
  // transfer j's rows lie 64 j rows past the first transfer's, clamped to the
  // last row of the matrix.
  uint32_t s_c = 0, s_buf = 0, back = 0;
  auto issue_scales = [&](uint32_t q) {
    uint8_t *st = smem + OFF_SC + s_buf + wave * 1024;
    const uint32_t ja = q % TA;
    uint32_t oa;
    if constexpr (!GROUPED) oa = min(lsa[0] + (ja * 64 + s_ar) * kscales, last_sa);
    else oa = lsa[ja];
    __builtin_amdgcn_global_load_lds((glb_void *)(p.a_s + s_c * 64 + oa - back), (lds_void *)(st + ja * 4096), 16, 0, 0);
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      const uint32_t jb = min(q + 4 * sb, (uint32_t)TB - 1);
      uint32_t ob;
      if constexpr (!GROUPED) ob = min(lsb[0] + (jb * 64 + s_bc) * kscales, last_sb);
      else ob = lsb[jb] + s_bc * kscales;
      __builtin_amdgcn_global_load_lds((glb_void *)(bs + s_c * 64 + ob - back), (lds_void *)(st + SC_B + jb * 4096), 16, 0, 0);
    }
  };
  // the lanes' step back for chunk c (a piece past the row's end: its first piece)
  auto scale_bases = [&](uint32_t c) { back = (c * 64 + pc * 16 < kscales) ? 0u : pc * 16; };

  const uint32_t wm = wave / NWN, wn = wave % NWN;
  const uint32_t l32 = lane % 32, lh = lane / 32;
  // LDS byte offsets of this lane's fragment rows: codes (inside a stage) and
  // scales (inside a chunk, without the step's piece)
  // A fragment i of wave row wm holds tile rows (NWM i + wm) * 32 .. + 31: with
  // two wave rows the 32-row groups alternate between them, so that a tile
  // whose rows end early leaves both about the same work
  uint32_t offA[FM][2], offB[FN][2], rowSA[FM], rowSB[FN], swA[FM], swB[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const uint32_t r = (NWM * i + wm) * 32 + l32;
#pragma unroll
    for (int h = 0; h < 2; ++h) offA[i][h] = r * 64 + (((2 * lh + h) ^ swz(r)) * 16);
    rowSA[i] = r * 64 + lh * 4;
    swA[i] = swz(r);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const uint32_t r = wn * WN + j * 32 + l32;
#pragma unroll
    for (int h = 0; h < 2; ++h) offB[j][h] = CODE_B + r * 64 + (((2 * lh + h) ^ swz(r)) * 16);
    rowSB[j] = SC_B + r * 64 + lh * 4;
    swB[j] = swz(r);
  }

  float16v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // fragments of half h of the code stage of global step g
  // (helpers take Frags<F, FB>: F, the number of this wave's A fragments that
  // hold rows of the tile (32-row groups past the last row are not read,
  // decoded or multiplied), and FB, the number of B fragments it multiplies)
  auto read_half = [&](auto f_tag, uint32_t stg, int h, u32x4 *xa, u32x4 *xb) {
    constexpr int F = decltype(f_tag)::F, FB = decltype(f_tag)::FB;
    const uint8_t *st = smem + stg;
#pragma unroll
    for (int i = 0; i < F; ++i) xa[i] = *reinterpret_cast<const u32x4 *>(st + offA[i][h]);
#pragma unroll
    for (int j = 0; j < FB; ++j) xb[j] = *reinterpret_cast<const u32x4 *>(st + offB[j][h]);
  };
  // scale dword of K step ks held in the chunk buffer at byte offset buf: piece (ks % 8) / 2 of
  // the row's 64 bytes, half ks % 2
  auto read_scales = [&](auto f_tag, uint32_t buf, uint32_t ks, uint32_t *xa, uint32_t *xb) {
    constexpr int F = decltype(f_tag)::F, FB = decltype(f_tag)::FB;
    const uint8_t *st = smem + OFF_SC + buf + (ks % 2) * 8;
    const uint32_t q = (ks % SC_STEPS) / 2;
#pragma unroll
    for (int i = 0; i < F; ++i) xa[i] = *reinterpret_cast<const uint32_t *>(st + rowSA[i] + ((q ^ swA[i]) * 16));
#pragma unroll
    for (int j = 0; j < FB; ++j) xb[j] = *reinterpret_cast<const uint32_t *>(st + rowSB[j] + ((q ^ swB[j]) * 16));
  };
  // scale pairs of one step: block b of the lane's four is pair b % 2, element b / 2
  auto pairs = [&](auto f_tag, const uint32_t *ya, const uint32_t *yb, half2v (*pa)[2], half2v (*pb)[2]) {
    constexpr int F = decltype(f_tag)::F, FB = decltype(f_tag)::FB;
#pragma unroll
    for (int i = 0; i < F; ++i) {
      pa[i][0] = scale_pair(ya[i]);
      pa[i][1] = scale_pair(ya[i] >> 8);
    }
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      pb[j][0] = scale_pair(yb[j]);
      pb[j][1] = scale_pair(yb[j] >> 8);
    }
  };
  // operands of MFMA sub-step t (0..7) of a K step: dword t % 4 of the
  // half-t/4 fragments, block b = t / 2 of the lane's four
  auto decode_step = [&](auto f_tag, int t, const u32x4 *xa, const u32x4 *xb, half2v (*pa)[2],
                         half2v (*pb)[2], half8v *oa8, half8v *ob8) {
    constexpr int F = decltype(f_tag)::F, FB = decltype(f_tag)::FB;
    const int b = t / 2;
#pragma unroll
    for (int i = 0; i < F; ++i) oa8[i] = decode8(xa[i][t % 4], pa[i][b % 2][b / 2]);
#pragma unroll
    for (int j = 0; j < FB; ++j) ob8[j] = decode8(xb[j][t % 4], pb[j][b % 2][b / 2]);
  };
  auto mfmas = [&](auto f_tag, const half8v *oa8, const half8v *ob8) {
    constexpr int F = decltype(f_tag)::F, FB = decltype(f_tag)::FB;
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < FB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ob8[j], oa8[i], acc[i][j], 0, 0, 0);
  };
  // one MFMA, then VPM VALU (a sub-step's decode spread over its MFMAs), F * FB
  // times; NV memory transfers and ND LDS reads spread evenly.  The reads of a
  // half step's operands go between its first MFMAs: issued as one burst right
  // after a barrier, the four waves' reads queue behind each other and hold up
  // the MFMAs (2-3% of the prefill GEMM's time)
  auto interleave = [&](auto f_tag, auto nv_tag, auto nd_tag) {
    constexpr int F = decltype(f_tag)::F, FB = decltype(f_tag)::FB;
    constexpr int NV = decltype(nv_tag)::value, NM = F * FB;
    constexpr int ND = decltype(nd_tag)::value;
    constexpr int VPM = (8 * (F + FB) + NM - 1) / NM;
#pragma unroll
    for (int k = 0; k < NM; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (ND > 0) {
        const int nd = ((k + 1) * ND) / NM - (k * ND) / NM;
#pragma unroll
        for (int v = 0; v < nd; ++v) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
      if constexpr (NV > 0 && NM >= NV) {
        if (k % (NM / NV) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      } else if constexpr (NV > 0) {
        // more transfers than MFMAs (a wave with one A fragment): spread evenly
        const int nk = ((k + 1) * NV) / NM - (k * NV) / NM;
#pragma unroll
        for (int v = 0; v < nk; ++v) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---------------------------------------------------------------- epilogue
  // The MFMAs take the weight fragment as their first operand, so accumulator
  // register r = 4q + e of lane (l32, lh) in a 32x32 tile holds output row l32,
  // column 8q + 4lh + e: each lane holds four runs of four consecutive columns
  // of one row.  Each wave stages RPP rows of one fragment row i at a time in
  // its own part of the code stage of the tile's last K step (free from the
  // mid-step barrier of that step until the next step's transfers, which a
  // workgroup barrier after the epilogue holds back), one 8-byte (bf16) or
  // 16-byte (float) LDS store per run, then reads them back 16 bytes per lane
  // and writes them out.  Staged rows are not padded (a fragment row of a
  // 256 x 256 tile fills a stage): the 16-byte chunks of staged row t are
  // rotated by t / (rows per 256 bytes), so that the rows of one store spread
  // over the banks.
  constexpr int ROW_ELEMS = WN_OUT;
  constexpr int ROW_BYTES = ROW_ELEMS * (int)sizeof(OutT);
  constexpr int CPR = ROW_BYTES / 16;  // 16-byte chunks per staged row
  constexpr int RPP = 4 * 32 * ROW_BYTES <= CODE_STAGE ? 32 : (4 * 16 * ROW_BYTES <= CODE_STAGE ? 16 : 8);
  constexpr int RW = ROW_BYTES >= 256 ? 1 : 256 / ROW_BYTES;  // staged rows per 256 bytes
  static_assert(ROW_BYTES % 16 == 0, "whole 16-byte chunks per staged row");
  static_assert(4 * RPP * ROW_BYTES <= CODE_STAGE, "epilogue staging must fit a stage");
  OutT *C = static_cast<OutT *>(p.c);
  auto epilogue = [&](uint32_t stg, uint32_t r0, uint32_t tn, uint32_t nf, auto split_tag) {
    // a column-split tile (split_tag true): one fragment row, row group 0 for
    // both wave rows, wave row wm holding half of its wave column's outputs
    constexpr bool SPL = decltype(split_tag)::value;
    // The lane's index, computed afresh here: lane-derived addresses kept live
    // across the K loop for the epilogue get spilled, and each reload waits for
    // every transfer in flight, including the next tile's first steps.
    uint32_t ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const uint32_t el32 = ln % 32, elh = ln / 32;
    uint8_t *slab = smem + stg + wave * RPP * ROW_BYTES;
    const uint32_t col0 = tn * BN_OUT + wn * WN_OUT + (SPL ? wm * (WN_OUT / 2) : 0u);
    // byte offset of 16-byte chunk c of staged row t
    auto at = [&](uint32_t t, uint32_t c) { return t * ROW_BYTES + ((c + t / RW) % CPR) * 16; };
    // output value of accumulator register r of fragments (i, j) (with the
    // gate: of gate fragment j and its up fragment j + HALF)
    constexpr int HOFF = SPL ? 1 : HALF;  // up fragment of gate fragment j: j + HOFF
    auto value = [&](int i, int j, int r) -> float {
      if constexpr (SILU) return silu(acc[i][j][r] * out_scale) * (acc[i][j + HOFF][r] * out_scale);
      else return acc[i][j][r] * out_scale;
    };
    constexpr int NJ = SPL ? (SILU ? 1 : 2) : (SILU ? HALF : FN);
    // 16-byte chunks of a staged row that hold outputs, and 16-element blocks
    constexpr int CPR_E = SPL ? CPR / 2 : CPR, BPR_E = (SPL ? ROW_ELEMS / 2 : ROW_ELEMS) / 16;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if ((uint32_t)i >= nf) break;  // rows past the tile's end: nothing to write
#pragma unroll
      for (int ps = 0; ps < 32 / RPP; ++ps) {
        // the lanes whose row falls in this pass store their runs
        if (el32 / RPP == (uint32_t)ps) {
          const uint32_t t = el32 % RPP;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              __builtin_amdgcn_sched_barrier(0);
              const float v0 = value(i, j, 4 * q), v1 = value(i, j, 4 * q + 1);
              const float v2 = value(i, j, 4 * q + 2), v3 = value(i, j, 4 * q + 3);
              if constexpr (sizeof(OutT) == 2) {
                // rounded to nearest even two at a time by the packed convert
                const float2v f01 = {v0, v1}, f23 = {v2, v3};
                const u32x2 pk = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f01, bf16x2v)),
                                  __builtin_bit_cast(uint32_t, __builtin_convertvector(f23, bf16x2v))};
                *reinterpret_cast<u32x2 *>(slab + at(t, 4 * j + q) + elh * 8) = pk;
              } else {
                const u32x4 fv = {f2u(v0), f2u(v1), f2u(v2), f2u(v3)};
                *reinterpret_cast<u32x4 *>(slab + at(t, 8 * j + 2 * q + elh)) = fv;
              }
            }
          }
        }
        // the slab is this wave's own: ordering inside the wave suffices (a
        // workgroup-scope fence would also wait for every load in flight)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const uint32_t rbase = r0 + (SPL ? 0u : (NWM * i + wm)) * 32 + ps * RPP;
        if constexpr (QOUT) {
          // NVFP4 output with the static global scale: 16-element blocks (four
          // staged chunks) one per lane at a time, the quantizer's arithmetic
          constexpr int NB = RPP * BPR_E;
#pragma unroll
          for (int b0 = 0; b0 < NB; b0 += 64) {
            const uint32_t b = b0 + ln, tr = b / BPR_E, bk = b % BPR_E;
            const uint32_t row = rbase + tr, col = col0 + bk * 16;
            if ((NB % 64 == 0 || b < (uint32_t)NB) && row < row_end && col < n_out) {
              float v[16];
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const u32x4 tv = *reinterpret_cast<const u32x4 *>(slab + at(tr, bk * 4 + k));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * k + e] = u2f(tv[e]);  // (by value: a bit cast
                                                                        // of a vector element
                                                                        // lvalue reads element 0)
              }
              float bmax = 0.0f;
#pragma unroll
              for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, fabsf(v[e]));
              const uint32_t sc = block_scale_code(bmax, h_six_g, h_inv_six_g);
              const float rr = 1.0f / (e4m3_value(sc) * h_g);
              uint32_t lo = 0, hi = 0;
              lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[0] * rr, v[1] * rr, 1.0f, 0);
              lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[2] * rr, v[3] * rr, 1.0f, 1);
              lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[4] * rr, v[5] * rr, 1.0f, 2);
              lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[6] * rr, v[7] * rr, 1.0f, 3);
              hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[8] * rr, v[9] * rr, 1.0f, 0);
              hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[10] * rr, v[11] * rr, 1.0f, 1);
              hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[12] * rr, v[13] * rr, 1.0f, 2);
              hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[14] * rr, v[15] * rr, 1.0f, 3);
              *reinterpret_cast<uint64_t *>(p.h_q + (int64_t)row * (n_out / 2) + col / 2) =
                  (uint64_t)lo | ((uint64_t)hi << 32);
              p.h_s[(int64_t)row * (n_out / 16) + col / 16] = (uint8_t)sc;
            }
          }
          __builtin_amdgcn_wave_barrier();
          continue;
        }
        // RPP rows x ROW_ELEMS outputs, 16 bytes (VEC elements) per lane-chunk:
        // every chunk of the pass is read from LDS first, then all are stored
        constexpr int VEC = 16 / (int)sizeof(OutT);
        constexpr int NCH = RPP * CPR_E, NIT = (NCH + 63) / 64;
        u32x4 chunk[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const uint32_t c = ln + it * 64;
          if (NCH % 64 == 0 || c < (uint32_t)NCH)
            chunk[it] = *reinterpret_cast<const u32x4 *>(slab + at(c / CPR_E, c % CPR_E));
        }
        // every row of the pass exists and every chunk is whole (interior
        // tiles): plain 16-byte stores at a per-lane base, no per-chunk checks
        if (VSTORE && rbase + RPP <= row_end && col0 + CPR_E * VEC <= n_out) {
          OutT *gb = C + (int64_t)rbase * p.ldc + col0;
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            const uint32_t c = ln + it * 64;
            if (NCH % 64 == 0 || c < (uint32_t)NCH)
              *reinterpret_cast<u32x4 *>(gb + (int64_t)(c / CPR_E) * p.ldc + (c % CPR_E) * VEC) = chunk[it];
          }
          __builtin_amdgcn_wave_barrier();
          continue;
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const uint32_t c = ln + it * 64;
          const uint32_t row = rbase + c / CPR_E, col = col0 + (c % CPR_E) * VEC;
          if ((NCH % 64 != 0 && c >= (uint32_t)NCH) || row >= row_end) continue;
          OutT *gp = C + (int64_t)row * p.ldc + col;
          if (VSTORE && col + VEC <= n_out) {
            *reinterpret_cast<u32x4 *>(gp) = chunk[it];
          } else {
            OutT sv[VEC];
            __builtin_memcpy(sv, &chunk[it], 16);
            for (int e = 0; e < VEC; ++e)
              if (col + e < n_out) gp[e] = sv[e];
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  };

  // ---------------------------------------------------------------- K loop
  // One stream of K steps over all tiles of the workgroup: global step g is K
  // step ks of tile i.  Software pipeline: while the MFMAs of sub-step t run,
  // the operands of sub-step t + 1 are decoded; the next step's first half is
  // read from LDS while this step's second half is multiplied.  Codes are
  // fetched AHEAD steps ahead (across a tile boundary: the next tile's first
  // steps); scale chunk c + 1 (or the next tile's chunk 0) during the first
  // four steps of chunk c.  Every step issues TN + NSC transfers (near the end
  // the last step's codes again, into a stage nobody reads any more; outside
  // the first four steps of a chunk the next chunk's scales again,
  // rewriting identical bytes), so at the mid-step barrier one wait count
  // leaves in flight only what was issued after the fetch of the next step.  At the last step of a
  // tile its epilogue runs, behind the already issued transfers of the next.
  uint32_t nrow0 = row0, nrow_end = row_end, ntile_n = tile_n;  // the tile after the current one
  if (my_tiles > 1) origin(1, &nrow0, &nrow_end, &ntile_n);
  // scale stream: chunk 0 of the first tile into buffer 0
  set_scale_target(row0, tile_n);
  scale_bases(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) issue_scales(j);
  // code stream: steps 0 .. AHEAD - 1 of the first tile into stages 0 ..
  // AHEAD - 1 (a short single tile reloads its last step into the stages past
  // it, which nobody reads; a walk of several tiles has at least 8 steps per
  // tile, so the stream runs at most into the next tile)
  set_fetch(row0, tile_n);
#pragma unroll
  for (int st = 0; st < AHEAD; ++st)
#pragma unroll
    for (int q = 0; q < TN; ++q) issue_code(st * CODE_STAGE, min((uint32_t)st, nsteps - 1), q);
  wait_vm<(AHEAD - 1) * TN>();
  // byte offsets of the code stages of global steps g - 1 (the stage the
  // fetch of step g + AHEAD fills), g, g + 1, ...: rotated after every step
  uint32_t sp[NSTAGE];
  sp[0] = (NSTAGE - 1) * CODE_STAGE;
#pragma unroll
  for (int k = 1; k < NSTAGE; ++k) sp[k] = (k - 1) * CODE_STAGE;
  uint32_t f_ks = AHEAD;  // the K step of the fetch tile the code stream fetches next
  uint32_t r_buf = 0;     // the scale buffer of the current step's chunk
  for (uint32_t ti = 0; ti < my_tiles; ++ti) {
    // this wave's A fragments that hold rows of the tile
    const uint32_t rows_in = min(row_end - min(row0, row_end), (uint32_t)BM);
    const uint32_t groups = (rows_in + 31) / 32;
    const uint32_t nf = groups > wm ? min((groups - wm + NWM - 1) / NWM, (uint32_t)FM) : 0u;
    auto run = [&](auto f_tag) {
    constexpr int F = decltype(f_tag)::F, FB = decltype(f_tag)::FB;
    const auto ft = f_tag;
    // the tile's first step: its data landed before the previous barrier
    // (fetched during the previous tile), or just above
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    u32x4 fa[FM], fb[FN];
    uint32_t sa[FM], sb[FN];
    if constexpr (F > 0) {
      read_half(ft, sp[1], 0, fa, fb);
      read_scales(ft, r_buf, 0, sa, sb);
    }
    wait_lgkm0();
    half2v spa[FM][2], spb[FN][2];
    half8v av[2][FM], bv[2][FN];
    if constexpr (F > 0) {
      pairs(ft, sa, sb, spa, spb);
      decode_step(ft, 0, fa, fb, spa, spb, av[0], bv[0]);
    }
    for (uint32_t ks = 0; ks < nsteps; ++ks) {
      // the code stream past its tile's end: the next tile (which becomes the
      // fetch tile) or, after the last tile, that tile's last step again
      if (f_ks >= nsteps) {
        if (ti + 1 < my_tiles) {
          f_ks -= nsteps;
          set_fetch(nrow0, ntile_n);
        } else {
          f_ks = nsteps - 1;
        }
      }
      // the scale stream, at a chunk's first step: the next chunk (of this
      // tile, or the next tile's first) into the other buffer, for all eight
      // steps of the chunk (the last four rewrite identical bytes), or, after
      // the last chunk of the last tile, this chunk again
      const uint32_t part = ks % SC_STEPS;
      if (part == 0) {
        const uint32_t chunk = ks / SC_STEPS;
        if (chunk + 1 < cpt) {
          s_c = chunk + 1;
          s_buf = r_buf ^ SC_CHUNK;
        } else if (ti + 1 < my_tiles) {
          s_c = 0;
          s_buf = r_buf ^ SC_CHUNK;
          set_scale_target(nrow0, ntile_n);
        } else {
          s_c = chunk;
          s_buf = r_buf;
        }
        scale_bases(s_c);
      }
      u32x4 ha[FM], hb[FN];
      if constexpr (F > 0) read_half(ft, sp[1], 1, ha, hb);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (F > 0) {
          mfmas(ft, av[t & 1], bv[t & 1]);
          if (t < 3) decode_step(ft, t + 1, fa, fb, spa, spb, av[(t + 1) & 1], bv[(t + 1) & 1]);
          else decode_step(ft, 4, ha, hb, spa, spb, av[0], bv[0]);
        }
#pragma unroll
        for (int q = (t * TN + 3) / 4; q < ((t + 1) * TN + 3) / 4; ++q) issue_code(sp[0], f_ks, q);
        if (t == 3) issue_scales(part % 4);
        if constexpr (F > 0) {
          if (t == 0) interleave(ft, std::integral_constant<int, ((1 * TN + 3) / 4 - (0 * TN + 3) / 4)>(), std::integral_constant<int, F + FB>());
          if (t == 1) interleave(ft, std::integral_constant<int, ((2 * TN + 3) / 4 - (1 * TN + 3) / 4)>(), std::integral_constant<int, 0>());
          if (t == 2) interleave(ft, std::integral_constant<int, ((3 * TN + 3) / 4 - (2 * TN + 3) / 4)>(), std::integral_constant<int, 0>());
          if (t == 3) interleave(ft, std::integral_constant<int, ((4 * TN + 3) / 4 - (3 * TN + 3) / 4) + NSC>(), std::integral_constant<int, 0>());
        }
      }
      // step g + 1 has landed: at most the transfers issued since the
      // fetch of step g + 1 (the last AHEAD - 1 steps' codes, and scales) remain
      wait_vm<(AHEAD - 1) * TN + NSC>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // the next step's first half (at a tile's last step: not used)
      const uint32_t nks = ks + 1 < nsteps ? ks + 1 : 0;
      const uint32_t nbuf = nks % SC_STEPS == 0 ? r_buf ^ SC_CHUNK : r_buf;  // a new chunk: the other buffer
      uint32_t na[FM], nb[FN];
      if constexpr (F > 0) {
        read_half(ft, sp[2], 0, fa, fb);
        read_scales(ft, nbuf, nks, na, nb);
      }
      half2v npa[FM][2], npb[FN][2];
      if constexpr (F > 0) {
#pragma unroll
        for (int t = 4; t < 8; ++t) {
          mfmas(ft, av[t & 1], bv[t & 1]);
          if (t < 7) {
            decode_step(ft, t + 1, ha, hb, spa, spb, av[(t + 1) & 1], bv[(t + 1) & 1]);
          } else {
            // keep the next step's operands from being used (and waited for) earlier
#pragma unroll
            for (int i = 0; i < F; ++i) asm volatile("" : "+v"(fa[i]), "+v"(na[i]));
#pragma unroll
            for (int j = 0; j < FB; ++j) asm volatile("" : "+v"(fb[j]), "+v"(nb[j]));
            pairs(ft, na, nb, npa, npb);
            decode_step(ft, 0, fa, fb, npa, npb, av[0], bv[0]);
          }
          if (t == 4) interleave(ft, std::integral_constant<int, 0>(), std::integral_constant<int, 2 * (F + FB)>());
          else interleave(ft, std::integral_constant<int, 0>(), std::integral_constant<int, 0>());
        }
      }
#pragma unroll
      for (int i = 0; i < F; ++i) {
        spa[i][0] = npa[i][0];
        spa[i][1] = npa[i][1];
      }
#pragma unroll
      for (int j = 0; j < FB; ++j) {
        spb[j][0] = npb[j][0];
        spb[j][1] = npb[j][1];
      }
      const uint32_t s0 = sp[0];
#pragma unroll
      for (int k = 0; k + 1 < NSTAGE; ++k) sp[k] = sp[k + 1];
      sp[NSTAGE - 1] = s0;
      r_buf = nbuf;
      ++f_ks;
    }
    };
    // A grouped tile holding a single 32-row group (an expert's last few rows)
    // splits columns instead of rows between the two wave rows: both take row
    // group 0, wave row wm half of its wave column's B fragments (without the
    // gate fragments 2 wm and 2 wm + 1; with it gate fragment wm and its up
    // fragment HALF + wm), so that wave row 1 does not idle at every barrier.
    // The per-wave offsets are remapped for the tile and restored after it.
    constexpr bool CAN_SPLIT = GROUPED && NWM == 2 && FN == 4;
    const bool split = CAN_SPLIT && groups == 1;
    uint32_t keep_a[2] = {0, 0}, keep_sa = 0, keep_b[2][2] = {{0, 0}, {0, 0}}, keep_sb[2] = {0, 0},
             keep_swb[2] = {0, 0};
    if constexpr (CAN_SPLIT) {
      if (split) {
        const uint32_t j0 = SILU ? wm : 2 * wm, j1 = SILU ? HALF + wm : 2 * wm + 1;
        auto pick = [&](const uint32_t (&v)[FN], uint32_t j) { return j == 0 ? v[0] : j == 1 ? v[1] : j == 2 ? v[2] : v[3]; };
        uint32_t ob0[FN], ob1[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          ob0[j] = offB[j][0];
          ob1[j] = offB[j][1];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) keep_a[h] = offA[0][h];
        keep_sa = rowSA[0];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          keep_b[j][0] = offB[j][0];
          keep_b[j][1] = offB[j][1];
          keep_sb[j] = rowSB[j];
          keep_swb[j] = swB[j];
        }
        const uint32_t nsb0 = pick(rowSB, j0), nsb1 = pick(rowSB, j1), nsw0 = pick(swB, j0), nsw1 = pick(swB, j1);
        offB[0][0] = pick(ob0, j0);
        offB[0][1] = pick(ob1, j0);
        offB[1][0] = pick(ob0, j1);
        offB[1][1] = pick(ob1, j1);
        rowSB[0] = nsb0;
        rowSB[1] = nsb1;
        swB[0] = nsw0;
        swB[1] = nsw1;
        // wave row 1's first fragment holds rows 32..63: 32 rows back (the
        // swizzle (r / 4) % 4 is the same 32 rows apart)
        if (wm == 1) {
          offA[0][0] -= 32 * 64;
          offA[0][1] -= 32 * 64;
          rowSA[0] -= 32 * 64;
        }
      }
    }

    // dispatch on F (uniform per wave; every variant runs the same barriers)
    if (CAN_SPLIT && split) run(Frags<1, 2>());
    else if (nf >= (uint32_t)FM) run(Frags<FM, FN>());
    else if (nf == 0) run(Frags<0, FN>());
    else if (nf == 1) run(Frags<1, FN>());
    else if constexpr (FM > 2) {
      if (nf == 2) run(Frags<2, FN>());
      else if constexpr (FM > 3) {
        if (nf == 3) run(Frags<3, FN>());
        else if constexpr (FM > 4) {
          if (nf == 4) run(Frags<4, FN>());
          else if constexpr (FM > 5) {
            if (nf == 5) run(Frags<5, FN>());
            else if constexpr (FM > 6) {
              if (nf == 6) run(Frags<6, FN>());
              else if constexpr (FM > 7) run(Frags<7, FN>());
            }
          }
        }
      }
    }

    // the tile is done: the next tile's first steps are already in flight
    wait_lgkm0();
    if (CAN_SPLIT && split) {
      epilogue(sp[0], row0, tile_n, 1u, std::true_type());
      if constexpr (CAN_SPLIT) {
#pragma unroll
        for (int h = 0; h < 2; ++h) offA[0][h] = keep_a[h];
        rowSA[0] = keep_sa;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          offB[j][0] = keep_b[j][0];
          offB[j][1] = keep_b[j][1];
          rowSB[j] = keep_sb[j];
          swB[j] = keep_swb[j];
        }
      }
    } else {
      epilogue(sp[0], row0, tile_n, nf, std::false_type());
    }
    // every wave's staging reads done before the next step's transfers rewrite
    // the stage (no wait for the transfers in flight: they fill other stages)
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    row0 = nrow0;
    row_end = nrow_end;
    tile_n = ntile_n;
    if (ti + 2 < my_tiles) origin(ti + 2, &nrow0, &nrow_end, &ntile_n);
  }
}

template <int BM, int BN, int WM, int WN, bool GROUPED, bool SILU, typename OutT>
hipError_t launch_cfg(const GemmParams &p, uint32_t grid, bool aligned, bool vstore,
                      hipStream_t stream) {
  constexpr int NT = Tile<BM, BN, WM, WN>::NT;
  if (aligned) {
    if (vstore)
      gemm_kernel<BM, BN, WM, WN, GROUPED, true, SILU, true, OutT><<<grid, NT, 0, stream>>>(p);
    else
      gemm_kernel<BM, BN, WM, WN, GROUPED, true, SILU, false, OutT><<<grid, NT, 0, stream>>>(p);
  } else {
    gemm_kernel<BM, BN, WM, WN, GROUPED, false, SILU, false, OutT><<<grid, NT, 0, stream>>>(p);
  }
  return hipGetLastError();
}

bool operands_aligned(const GemmParams &p) {
  auto al = [](const void *q, uintptr_t a) { return ((uintptr_t)q & (a - 1)) == 0; };
  return p.K % BK == 0 && al(p.a_q, 16) && al(p.a_s, 8) && al(p.b_q, 16) && al(p.b_s, 8) &&
         p.b_mstride_q % 16 == 0 && p.b_mstride_s % 8 == 0;
}

// The direct-to-LDS kernel needs whole 256-element K chunks and per-lane byte
// offsets that fit 32 bits (rows x K/2 for the codes of either operand).
bool dma_ok(const GemmParams &p, uint64_t a_rows) {
  const uint64_t kb = p.K / 2;
  auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
  return p.K % 256 == 0 && a_rows * kb < (1ull << 32) && (uint64_t)p.N * kb < (1ull << 32) &&
         al16(p.a_q) && al16(p.a_s) && al16(p.b_q) && al16(p.b_s) && p.b_mstride_q % 16 == 0 &&
         p.b_mstride_s % 16 == 0;
}

// Dense launches with whole 8-step scale chunks (K % 1024 == 0) run one
// workgroup per compute unit, each walking its tiles with the next tile's
// first K steps fetched during the current tile's last ones; otherwise one
// workgroup per tile.  The CU count is a multiple of 8, which keeps every
// workgroup's tiles on one XCD.  A product with at most half as many tiles as
// compute units launches two workgroups per tile, one per half of its rows
// (the kernel splits the tiles of a last round that is at most half full).
uint32_t dense_grid(const GemmParams &p, uint32_t tiles, uint32_t bm) {
  const uint32_t g = device_cu_count() & ~7u;
  if (g != 0 && 2 * tiles <= g && p.M > bm / 2) return 2 * tiles;
  if ((p.K / 128) % 8 != 0) return tiles;
  return g == 0 || tiles <= g ? tiles : g;
}

template <int BM, bool GROUPED, bool SILU, bool VSTORE, typename OutT, bool QOUT = false, int NWM = 2,
          int BN = 256>
hipError_t launch_dma(const GemmParams &p, uint32_t grid, hipStream_t stream) {
  gemm_dma_kernel<BM, GROUPED, SILU, VSTORE, OutT, QOUT, NWM, BN><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

// Tile width for dense products of at most 128 rows: one tile row, so the
// column tiles are the whole schedule, one workgroup per compute unit.  A
// product whose 256-column tiles leave a partly filled last round (run as row
// halves, at about 0.8 of a round: a half tile still decodes most of a full
// tile's operands) can take 320-column tiles (2 x 2 waves of 64 x 160) in
// fewer rounds: lm_head 128 x 151936 needs 594 tiles of 256 (2.32 rounds, run
// in about 2.8) or 475 of 320 (two rounds).  The cost compared is rounds x
// width; 320 only with more than 32 rows (with fewer, a 2 x 2 tile leaves its
// second wave row idle).
int skinny_tile_width(const GemmParams &p) {
  const uint32_t cu = device_cu_count() & ~7u;
  if (cu == 0 || p.M <= 32) return 256;
  const bool halves = p.M > 64, persistent = (p.K / 128) % 8 == 0;
  auto cost = [&](uint32_t bn) {
    const uint32_t tiles = (p.N + bn - 1) / bn;
    double rounds;
    if (2 * tiles <= cu && halves) {
      rounds = 0.8;
    } else if (tiles <= cu) {
      rounds = 1.0;
    } else {
      const uint32_t full = tiles / cu, rem = tiles % cu;
      rounds = full + (rem == 0 ? 0.0 : (persistent && 2 * rem <= cu && halves ? 0.8 : 1.0));
    }
    return rounds * bn;
  };
  return cost(320) < 0.95 * cost(256) ? 320 : 256;
}

// Tile height for the grouped GEMM from the mean rows per expert m = R / E.
// Per-expert counts of a top-k router spread like a Poisson count around m,
// and an expert with n rows costs ceil(n / BM) tiles of BM rows.  Shorter
// tiles waste fewer rows but cost more per row: the decode work per MFMA
// grows as BM shrinks, and a K step has fewer MFMAs to hide it under.
// Relative cost per computed row, measured on MI355X with 2 x 2 waves: 1.5
// (128 rows), 1.2 (192), 1.0 (256); the 1 x 4 waves that 128- and 192-row
// tiles now use take 2-4% less time on the 512-expert workload's GEMMs.  The expected cost
// of each height is estimated over 32 quantiles of a normal N(m, m) and the
// cheapest height wins.
int grouped_tile_rows(uint32_t R, uint32_t E) {
  const double m = (double)R / (double)E, sd = m > 1.0 ? __builtin_sqrt(m) : 1.0;
  // upper half of the standard normal quantiles at (i + 0.5) / 32
  static const double z[16] = {0.0392, 0.1178, 0.1971, 0.2777, 0.3601, 0.4451, 0.5334, 0.6261,
                               0.7245, 0.8305, 0.9468, 1.0775, 1.2299, 1.4178, 1.6759, 2.1539};
  static const int height[3] = {128, 192, 256};
  static const double row_cost[3] = {1.5, 1.2, 1.0};
  int best = 128;
  double best_cost = 1e300;
  for (int h = 0; h < 3; ++h) {
    double tiles = 0.0;
    for (int i = 0; i < 16; ++i)
      for (int sgn = -1; sgn <= 1; sgn += 2) {
        const double n = m + sgn * z[i] * sd;
        tiles += n > 0.0 ? __builtin_ceil(n / height[h]) : 0.0;
      }
    const double cost = tiles / 32.0 * height[h] * row_cost[h];
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = height[h];
    }
  }
  return best;
}

bool stores_aligned(const GemmParams &p, OutType out) {
  const int64_t es = out == OutType::BF16 ? 2 : 4;
  return ((uintptr_t)p.c & 15u) == 0 && (p.ldc * es) % 16 == 0;
}

}  // namespace

bool grouped_nvfp4_out_supported(const GemmParams &p) {
  return operands_aligned(p) && dma_ok(p, p.a_rows) && (p.N / 2) % 16 == 0 &&
         ((uintptr_t)p.h_q & 7u) == 0;
}

hipError_t launch_gemm(const GemmParams &p, OutType out, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  constexpr int BM = 256, BN = 256;
  const uint32_t grid = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const bool al = operands_aligned(p), vs = stores_aligned(p, out);
  if (al && dma_ok(p, p.M)) {
    // skinny products (decode batches, lm_head) take the 128-row tile: half the
    // MFMA work of a mostly empty 256-row tile, twice the workgroups.  Its four
    // waves sit side by side (1 x 4, each over all 128 rows and 64 columns):
    // every B fragment is decoded by one wave only, and a tile split into row
    // halves decodes 4 fragments per 4 MFMAs instead of 5 (2 x 2 waves).
    // Measured against 2 x 2 on one host: lm_head 128x151936x2048 97.5 -> 95.5
    // us; M x 32768 x 4096 at M = 32 / 64 / 128: 44 -> 35, 47 -> 42, 51 -> 45 us.
    // Where 320-column tiles take fewer rounds (skinny_tile_width), those run
    // instead, 2 x 2: lm_head 101 -> 96 us, bit-identical output.
    auto go = [&](auto bm_tag, auto bn_tag) -> hipError_t {
      constexpr int TBM = decltype(bm_tag)::value, TBN = decltype(bn_tag)::value;
      const uint32_t tiles = ((p.N + TBN - 1) / TBN) * ((p.M + TBM - 1) / TBM);
      const uint32_t g = dense_grid(p, tiles, TBM);
      constexpr int W = (TBM == 128 && TBN == 256) ? 1 : 2;
      if (out == OutType::BF16)
        return vs ? launch_dma<TBM, false, false, true, uint16_t, false, W, TBN>(p, g, stream)
                  : launch_dma<TBM, false, false, false, uint16_t, false, W, TBN>(p, g, stream);
      return vs ? launch_dma<TBM, false, false, true, float, false, W, TBN>(p, g, stream)
                : launch_dma<TBM, false, false, false, float, false, W, TBN>(p, g, stream);
    };
    if (p.M > 128) return go(std::integral_constant<int, BM>(), std::integral_constant<int, BN>());
    if (skinny_tile_width(p) == 320)
      return go(std::integral_constant<int, 128>(), std::integral_constant<int, 320>());
    return go(std::integral_constant<int, 128>(), std::integral_constant<int, 256>());
  }
  return out == OutType::BF16
             ? launch_cfg<BM, BN, 128, 128, false, false, uint16_t>(p, grid, al, vs, stream)
             : launch_cfg<BM, BN, 128, 128, false, false, float>(p, grid, al, vs, stream);
}

hipError_t launch_grouped_gemm(const GemmParams &p, uint32_t R, OutType out, Epilogue epi,
                               hipStream_t stream) {
  if (R == 0) return hipSuccess;
  constexpr int BN = 256;
  const bool silu = epi == Epilogue::SiluGate || epi == Epilogue::SiluGateNvfp4;
  const uint32_t n_out = silu ? p.N / 2 : p.N;
  const uint32_t bn_out = silu ? BN / 2 : BN;
  const uint32_t tiles_n = (n_out + bn_out - 1) / bn_out;
  // sum_e ceil(n_e / BM) <= R / BM + E
  auto grid_for = [&](uint32_t bm) {
    return (uint32_t)(((uint64_t)(R + bm - 1) / bm + p.E) * tiles_n);
  };
  const bool al = operands_aligned(p), vs = stores_aligned(p, out);
  const bool qout = epi == Epilogue::SiluGateNvfp4;
  if (qout && !(al && dma_ok(p, p.a_rows))) return hipErrorNotSupported;
  if (al && dma_ok(p, p.a_rows)) {
    const int bm = grouped_tile_rows(R, p.E);
    // M tiles rounded up to a multiple of 8 (the kernel's XCD-major tile order);
    // one workgroup per N tile, or per pair of them when the kernel walks
    const uint64_t mt = ((uint64_t)R + bm - 1) / bm + p.E;
    const uint32_t tpw = grouped_walk(bm, silu, p.K, n_out, bn_out) ? 2u : 1u;
    const uint32_t grid = (uint32_t)(((mt + 7) & ~(uint64_t)7) * tiles_n / tpw);
    auto go = [&](auto bm_tag) -> hipError_t {
      constexpr int TBM = decltype(bm_tag)::value;
      // 128- and 192-row tiles: four waves side by side (1 x 4), each over all
      // of the tile's rows, so a tile holding an odd number of 32-row groups
      // keeps every wave busy (2 x 2 waves split 5 groups 3 + 2, the cost of
      // 6); 256-row tiles stay 2 x 2, which leaves the registers for the
      // pipeline (eight A fragments per wave would not fit)
      constexpr int W = TBM == 256 ? 2 : 1;
      if (qout) return launch_dma<TBM, true, true, false, float, true>(p, grid, stream);
      if (silu)
        return out == OutType::BF16
                   ? (vs ? launch_dma<TBM, true, true, true, uint16_t, false, W>(p, grid, stream)
                         : launch_dma<TBM, true, true, false, uint16_t, false, W>(p, grid, stream))
                   : (vs ? launch_dma<TBM, true, true, true, float, false, W>(p, grid, stream)
                         : launch_dma<TBM, true, true, false, float, false, W>(p, grid, stream));
      return out == OutType::BF16
                 ? (vs ? launch_dma<TBM, true, false, true, uint16_t, false, W>(p, grid, stream)
                       : launch_dma<TBM, true, false, false, uint16_t, false, W>(p, grid, stream))
                 : (vs ? launch_dma<TBM, true, false, true, float, false, W>(p, grid, stream)
                       : launch_dma<TBM, true, false, false, float, false, W>(p, grid, stream));
    };
    if (bm == 256) return go(std::integral_constant<int, 256>());
    if (bm == 192) return go(std::integral_constant<int, 192>());
    return go(std::integral_constant<int, 128>());
  }
  constexpr int BM = 128;
  const uint32_t grid = grid_for(BM);
  if (silu)
    return out == OutType::BF16
               ? launch_cfg<BM, BN, 64, 128, true, true, uint16_t>(p, grid, al, vs, stream)
               : launch_cfg<BM, BN, 64, 128, true, true, float>(p, grid, al, vs, stream);
  return out == OutType::BF16
             ? launch_cfg<BM, BN, 64, 128, true, false, uint16_t>(p, grid, al, vs, stream)
             : launch_cfg<BM, BN, 64, 128, true, false, float>(p, grid, al, vs, stream);
}

}  // namespace nvfp4
