// fp8_gemm.hip -- FP8 (E4M3) W8A8 GEMM with per-tensor scales on gfx950.
//
// QAD tutorial (Model-Optimizer, Qwen3.6-35B-A3B W4A4), table of quantized
// tensors: next to the NVFP4 experts the attention projections stay FP8 W8A8;
// format-selection guide, section 1: FP8 is W8A8 with one scale per tensor.
// So C = (a_g * b_g) * sum_k e4m3(A[m][k]) * e4m3(B[n][k]) with float32
// accumulation, A [M][K] the activations and B [N][K] the weight, both
// row-major E4M3FN bytes.
//
// Design (CDNA4): E4M3 is a native MFMA operand type, so there is no decode.
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP8 E4M3 and unit
//    block scales (E8M0 127 = 2^0): 64 K elements per instruction, 32 bytes
//    per lane per operand.  The per-tensor scales are applied once, in the
//    epilogue.
//  * The K order inside a 64-element step is the same for both operands (lane
//    half h supplies bytes [32h, 32h + 32) of its row of A and of B), so the
//    dot product pairs the right elements whatever order the instruction sums
//    them in.
//  * 256-column tiles, BM = 256 (or 128 for short M) rows, four waves of
//    (BM/2) x 128: each lane holds (BM/64) x 4 accumulators of 32 x 32.
//  * Operands go from global memory straight into LDS (global_load_lds_dwordx4:
//    64 lanes x 16 bytes into 1 KB of consecutive LDS): four stages of one
//    64-byte K step per row (the 64-byte row swizzle of the NVFP4 kernels
//    keeps the 16-byte fragment reads free of bank conflicts), fetched four
//    steps ahead.  Every step issues the same transfers (at the end the last
//    step again, into a stage nobody reads), so one wait count serves every
//    step.
//  * Fragments are double buffered in registers: the LDS reads of step s + 1
//    are issued first and complete behind the 16 MFMAs of step s, over which
//    the transfers of step s + 4 are spread.  (Spreading the reads over the
//    MFMAs too, as the NVFP4 kernel does with its half-step reads, cost 6.5%:
//    here they are a whole step ahead of their use.)
//  * Tiles are ordered XCD-aware (dense_tile).  The MFMAs take the weight
//    fragment first, so each lane holds runs of four output columns of one
//    row; the epilogue stages each wave's 32-row slab through LDS with 8- or
//    16-byte stores so that global stores are 16 bytes per lane.
//  * K % 128 != 0 or row offsets beyond 32 bits take a plain kernel: direct
//    16-byte global loads into registers, one 32 x 32 tile per wave.
#include "nvfp4_common.hpp"
#include "nvfp4_format.hpp"
#include "nvfp4_kernels.hpp"

#include <type_traits>

namespace nvfp4 {

namespace {

typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int KS = 64;  // K elements (bytes) per step

__device__ __forceinline__ float16v mfma_fp8(i32x8 a, i32x8 b, float16v c) {
  // formats 0/0: both operands FP8 E4M3; scales 127: 2^0 for every block
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <typename OutT>
__device__ __forceinline__ OutT to_out(float v);
template <>
__device__ __forceinline__ float to_out<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t to_out<uint16_t>(float v) { return (uint16_t)float_to_bf16_bits(v); }

template <int BM, bool VSTORE, typename OutT>
__global__ __launch_bounds__(256, 1) void fp8_gemm_dma_kernel(Fp8GemmParams p) {
  constexpr int BN = 256, WM = BM / 2, WN = 128, FM = WM / 32, FN = WN / 32;
  static_assert(BM == 128 || BM == 256, "tile height");
  constexpr int TA = BM / 64, TB = BN / 64, TN = TA + TB;  // transfers per wave per step
  constexpr int OFF_B = BM * KS, STAGE = (BM + BN) * KS, NST = 4;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * STAGE];

  const uint32_t tid = threadIdx.x;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const uint32_t K = p.K, S = K / KS;
  const uint32_t tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  uint32_t tm, tn;
  dense_tile(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const uint32_t row0 = tm * BM, col0 = tn * BN;

  // Transfer j of an operand covers LDS slots j * 256 + tid: tile row
  // j * 64 + tid / 4, physical 16-byte piece tid % 4, which holds logical piece
  // pc = (tid % 4) ^ swz(row) (the same for every j).  Rows past the end of a
  // matrix reload its last row (never stored).  Offsets fit 32 bits (host).
  const uint32_t pc = (tid % 4) ^ swz(tid / 4);
  uint32_t oa[TA], ob[TB];
#pragma unroll
  for (int j = 0; j < TA; ++j) oa[j] = min(row0 + j * 64 + tid / 4, p.M - 1) * K + pc * 16;
#pragma unroll
  for (int j = 0; j < TB; ++j) ob[j] = min(col0 + j * 64 + tid / 4, p.N - 1) * K + pc * 16;
  auto issue = [&](uint32_t buf, uint32_t ks, int q) {
    uint8_t *st = smem + buf * STAGE + wave * 1024;
    if (q < TA)
      __builtin_amdgcn_global_load_lds((glb_void *)(p.a_q + ks * KS + oa[q]), (lds_void *)(st + q * 4096), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((glb_void *)(p.b_q + ks * KS + ob[q - TA]),
                                       (lds_void *)(st + OFF_B + (q - TA) * 4096), 16, 0, 0);
  };

  // this lane's fragment rows: pieces 2 lh and 2 lh + 1 of row r
  const uint32_t wm = wave / 2, wn = wave % 2;
  const uint32_t l32 = lane % 32, lh = lane / 32;
  uint32_t fa[FM][2], fb[FN][2];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const uint32_t r = wm * WM + i * 32 + l32;
#pragma unroll
    for (int h = 0; h < 2; ++h) fa[i][h] = r * KS + (((2 * lh + h) ^ swz(r)) * 16);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const uint32_t r = wn * WN + j * 32 + l32;
#pragma unroll
    for (int h = 0; h < 2; ++h) fb[j][h] = OFF_B + r * KS + (((2 * lh + h) ^ swz(r)) * 16);
  }
  auto read = [&](uint32_t buf, i32x8 *xa, i32x8 *xb) {
    const uint8_t *st = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      xa[i] = join(*reinterpret_cast<const u32x4 *>(st + fa[i][0]), *reinterpret_cast<const u32x4 *>(st + fa[i][1]));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      xb[j] = join(*reinterpret_cast<const u32x4 *>(st + fb[j][0]), *reinterpret_cast<const u32x4 *>(st + fb[j][1]));
  };

  float16v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---------------------------------------------------------------- K loop
  // Step s: stage s + 1 has landed (own transfers waited, then the barrier for
  // everyone's); the fragments of stage s are in registers; buffer s % 4 is
  // free (its reads were waited for before the barrier) and receives step
  // s + 4.  Before the wait, steps s + 1 .. s + 3 are in flight.
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int q = 0; q < TN; ++q) issue(st, min((uint32_t)st, S - 1), q);
  wait_vm<3 * TN>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  i32x8 xa[2][FM], xb[2][FN];
  read(0, xa[0], xb[0]);

  auto step = [&](uint32_t s, auto cur_tag) {
    constexpr int C = decltype(cur_tag)::value, NX = C ^ 1;
    wait_vm<2 * TN>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint32_t ks = min(s + NST, S - 1);
    // the next step's fragments: issued first, they complete behind the MFMAs
    read((s + 1) % NST, xa[NX], xb[NX]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < TN; ++q) issue(s % NST, ks, q);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma_fp8(xb[C][j], xa[C][i], acc[i][j]);
    // the transfers spread over the MFMAs, at most one after each
    constexpr int NM = FM * FN;
    static_assert(TN <= NM, "interleave shares");
#pragma unroll
    for (int k = 0; k < NM; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if ((k + 1) * TN / NM - k * TN / NM == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (uint32_t s = 0; s < S; s += 2) {
    step(s, std::integral_constant<int, 0>());
    step(s + 1, std::integral_constant<int, 1>());
  }
  // every transfer (including the reloads into unread stages) has landed and
  // every wave is past its last read: all of LDS is free for the epilogue
  wait_vm<0>();
  wait_lgkm0();
  __syncthreads();

  // ---------------------------------------------------------------- epilogue
  // The MFMAs take the weight fragment first, so accumulator register
  // r = 4q + e of lane (l32, lh) in a 32 x 32 tile holds output row l32, column
  // 8q + 4lh + e: four runs of four consecutive columns of one row.  Each wave
  // stages one fragment row (32 rows x 128 columns) at a time in its own part of
  // LDS, one 8-byte (bf16) or 16-byte (float) store per run, the 16-byte chunks
  // of staged row t rotated by t / (rows per 256 bytes) so that the rows of one
  // store spread over the banks, then reads every chunk back and writes it out
  // 16 bytes per lane.
  const float scale = (*p.a_g) * (*p.b_g);
  constexpr int ROW_BYTES = WN * (int)sizeof(OutT);
  constexpr int CPR = ROW_BYTES / 16;  // 16-byte chunks per staged row
  constexpr int RW = ROW_BYTES >= 256 ? 1 : 256 / ROW_BYTES;
  static_assert(4 * 32 * ROW_BYTES <= NST * STAGE, "epilogue staging must fit");
  uint8_t *slab = smem + wave * 32 * ROW_BYTES;
  auto at = [&](uint32_t t, uint32_t c) { return t * ROW_BYTES + ((c + t / RW) % CPR) * 16; };
  OutT *Cp = static_cast<OutT *>(p.c);
  const uint32_t ccol0 = col0 + wn * WN;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v0 = acc[i][j][4 * q] * scale, v1 = acc[i][j][4 * q + 1] * scale;
        const float v2 = acc[i][j][4 * q + 2] * scale, v3 = acc[i][j][4 * q + 3] * scale;
        if constexpr (sizeof(OutT) == 2) {
          // rounded to nearest even two at a time by the packed convert
          const float2v f01 = {v0, v1}, f23 = {v2, v3};
          const u32x2 pk = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f01, bf16x2v)),
                            __builtin_bit_cast(uint32_t, __builtin_convertvector(f23, bf16x2v))};
          *reinterpret_cast<u32x2 *>(slab + at(l32, 4 * j + q) + lh * 8) = pk;
        } else {
          const u32x4 fv = {f2u(v0), f2u(v1), f2u(v2), f2u(v3)};
          *reinterpret_cast<u32x4 *>(slab + at(l32, 8 * j + 2 * q + lh)) = fv;
        }
      }
    }
    // the slab is this wave's own: ordering inside the wave suffices
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    constexpr int VEC = 16 / (int)sizeof(OutT);
    constexpr int NCH = 32 * CPR, NIT = NCH / 64;
    static_assert(NCH % 64 == 0, "whole rounds of chunks");
    const uint32_t rbase = row0 + wm * WM + i * 32;
    u32x4 chunk[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const uint32_t c = lane + it * 64;
      chunk[it] = *reinterpret_cast<const u32x4 *>(slab + at(c / CPR, c % CPR));
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const uint32_t c = lane + it * 64;
      const uint32_t row = rbase + c / CPR, col = ccol0 + (c % CPR) * VEC;
      if (row >= p.M) continue;
      OutT *gp = Cp + (int64_t)row * p.ldc + col;
      if (VSTORE && col + VEC <= p.N) {
        *reinterpret_cast<u32x4 *>(gp) = chunk[it];
      } else {
        OutT sv[VEC];
        __builtin_memcpy(sv, &chunk[it], 16);
        for (int e = 0; e < VEC; ++e)
          if (col + e < p.N) gp[e] = sv[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Plain kernel (any K % 16 == 0, 64-bit offsets): a 64 x 64 tile per
// workgroup, one 32 x 32 MFMA tile per wave, operands loaded from global
// memory into registers 16 bytes at a time (zero past K).
template <typename OutT>
__global__ __launch_bounds__(256) void fp8_gemm_plain_kernel(Fp8GemmParams p) {
  const uint32_t tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const uint32_t l32 = lane % 32, lh = lane / 32;
  const uint32_t tiles_n = (p.N + 63) / 64;
  const uint32_t row0 = (blockIdx.x / tiles_n) * 64 + (wave / 2) * 32;
  const uint32_t col0 = (blockIdx.x % tiles_n) * 64 + (wave % 2) * 32;
  const uint64_t K = p.K;
  const uint8_t *ar = p.a_q + (uint64_t)min(row0 + l32, p.M - 1) * K;
  const uint8_t *br = p.b_q + (uint64_t)min(col0 + l32, p.N - 1) * K;
  float16v acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (uint64_t k0 = 0; k0 < K; k0 += KS) {
    u32x4 a[2], b[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint64_t k = k0 + 32 * lh + 16 * h;
      const bool in = k < K;  // K % 16 == 0: a 16-byte piece is all in or all out
      a[h] = in ? *reinterpret_cast<const u32x4 *>(ar + k) : (u32x4){0, 0, 0, 0};
      b[h] = in ? *reinterpret_cast<const u32x4 *>(br + k) : (u32x4){0, 0, 0, 0};
    }
    acc = mfma_fp8(join(a[0], a[1]), join(b[0], b[1]), acc);
  }
  const float scale = (*p.a_g) * (*p.b_g);
  OutT *Cp = static_cast<OutT *>(p.c);
  const uint32_t col = col0 + l32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t row = row0 + 8 * (r / 4) + 4 * lh + (r % 4);
    if (row < p.M && col < p.N) Cp[(int64_t)row * p.ldc + col] = to_out<OutT>(acc[r] * scale);
  }
}

template <int BM, typename OutT>
hipError_t launch_dma(const Fp8GemmParams &p, bool vstore, hipStream_t stream) {
  const uint32_t grid = ((p.M + BM - 1) / BM) * ((p.N + 255) / 256);
  if (vstore)
    fp8_gemm_dma_kernel<BM, true, OutT><<<grid, 256, 0, stream>>>(p);
  else
    fp8_gemm_dma_kernel<BM, false, OutT><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

template <typename OutT>
hipError_t launch_typed(const Fp8GemmParams &p, hipStream_t stream) {
  const bool vstore = ((uintptr_t)p.c % 16 == 0) && (p.ldc * (int64_t)sizeof(OutT)) % 16 == 0;
  if (fp8_gemm_dma_ok(p)) return p.M <= 128 ? launch_dma<128, OutT>(p, vstore, stream)
                                            : launch_dma<256, OutT>(p, vstore, stream);
  const uint64_t grid = (uint64_t)((p.M + 63) / 64) * ((p.N + 63) / 64);
  if (grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
  fp8_gemm_plain_kernel<OutT><<<(uint32_t)grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

// The direct-to-LDS kernel needs whole pairs of 64-element K steps, 16-byte
// aligned rows and per-lane byte offsets that fit 32 bits.
bool fp8_gemm_dma_ok(const Fp8GemmParams &p) {
  auto al16 = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
  return p.K % 128 == 0 && (uint64_t)p.M * p.K < (1ull << 32) && (uint64_t)p.N * p.K < (1ull << 32) &&
         al16(p.a_q) && al16(p.b_q);
}

hipError_t launch_fp8_gemm(const Fp8GemmParams &p, OutType out, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  return out == OutType::F32 ? launch_typed<float>(p, stream) : launch_typed<uint16_t>(p, stream);
}

}  // namespace nvfp4
