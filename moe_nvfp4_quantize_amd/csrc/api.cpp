// api.cpp -- the C ABI declared in include/nvfp4.h: argument validation on the
// host, the gfx950 device check, and dispatch to the kernel launchers.
//
// Validation runs before any HIP call, so an invalid request returns
// NVFP4_ERR_INVALID_ARG without touching the device (and works on a machine with
// no GPU at all).
#include "nvfp4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "nvfp4_kernels.hpp"

namespace {

using namespace nvfp4;

constexpr int64_t kI32Max = 0x7FFFFFFF;
constexpr int kMaxDevices = 64;
// 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_arch_ok[kMaxDevices];

nvfp4_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NVFP4_ERR_HIP;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? NVFP4_OK : NVFP4_ERR_UNSUPPORTED;
}

nvfp4_status from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

bool valid_dtype(nvfp4_dtype t) { return t == NVFP4_F32 || t == NVFP4_BF16; }
size_t dtype_size(nvfp4_dtype t) { return t == NVFP4_F32 ? 4 : 2; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// batched: per-matrix amax partials; single (batch 0 here means "single
// tensor"): the resident-kernel state followed by the partials
size_t quant_ws(int64_t batch, int64_t rows, int64_t cols, bool single) {
  if (batch <= 0 || rows < 0 || cols <= 0 || cols % 16 != 0) return 0;
  const uint64_t units = (uint64_t)rows * (uint64_t)(cols / 16);
  const size_t partials = round_up((size_t)batch * quantize_partials_per_matrix(units) * sizeof(float), 256);
  return single ? kResidentStateBytes + partials : partials;
}

// shape rules shared by the quantize entry points
bool quant_shape_ok(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0 || cols % 16 != 0) return false;
  if (rows > kI32Max || cols > kI32Max) return false;
  return rows * (cols / 16) <= kI32Max;
}

QuantParams make_quant(const void *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *q,
                       uint8_t *s, float *g, void *ws, int static_global) {
  QuantParams p{};
  p.x = x;
  p.ld = ld;
  p.x_mstride = rows * ld;
  p.rows = (uint32_t)rows;
  p.nbpr = (uint32_t)(cols / 16);
  p.units = (uint32_t)(rows * (cols / 16));
  p.div_nbpr = FastDiv(p.nbpr);
  p.q = q;
  p.s = s;
  p.g = g;
  p.q_mstride = rows * (cols / 2);
  p.s_mstride = rows * (cols / 16);
  p.partials = static_cast<float *>(ws);
  p.P = quantize_partials_per_matrix(p.units);
  p.static_global = static_global;
  return p;
}

// Dynamic quantize on the device (validated arguments; workspace holds the
// resident-kernel state followed by the amax partials).
nvfp4_status quantize_impl(const void *x, nvfp4_dtype x_type, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t *q, uint8_t *s, float *g, int static_global, void *workspace,
                           hipStream_t stream) {
  const bool vec = aligned16(x) && (ld_x * (int64_t)dtype_size(x_type)) % 16 == 0;
  ResidentState *rs = static_cast<ResidentState *>(workspace);
  void *partials = workspace ? static_cast<uint8_t *>(workspace) + kResidentStateBytes : nullptr;
  QuantParams p = make_quant(x, rows, cols, ld_x, q, s, g, partials, static_global ? 1 : 0);
  return from_hip(launch_quantize(p, x_type == NVFP4_BF16, vec, 1, rs, stream));
}

// ---------------------------------------------- allocation-free quantize
// Scratch of nvfp4_quantize_noalloc: the resident kernel's arrival state and
// the amax partials (at most kMaxPartials per tensor, whatever its size).
// Every GPU the library runs on holds its own copy until the process ends.
constexpr size_t kScratchBytes = kResidentStateBytes + (kMaxPartials * sizeof(float) + 255) / 256 * 256;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this device's scratch (the array's host-side name is a
// stand-in that kernels cannot use), looked up once per device with that
// device current.  The first call on a device also zero-fills it with a
// kernel on the caller's stream, ordered before that call's own kernels;
// after that every completed call leaves the arrival state ready for the
// next.
std::atomic<uintptr_t> g_scratch[kMaxDevices];

__global__ void zero_scratch_kernel(uint32_t *p, uint32_t words) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) p[i] = 0u;
}

nvfp4_status device_scratch(void **out, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
  uintptr_t a = g_scratch[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return NVFP4_ERR_HIP;
    zero_scratch_kernel<<<1, 256, 0, stream>>>(static_cast<uint32_t *>(ptr), (uint32_t)(kScratchBytes / 4));
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
    a = reinterpret_cast<uintptr_t>(ptr);
    g_scratch[dev].store(a, std::memory_order_release);
  }
  *out = reinterpret_cast<void *>(a);
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char *nvfp4_status_string(nvfp4_status status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_INVALID_ARG: return "NVFP4_ERR_INVALID_ARG: invalid argument";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED: unsupported device or request";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP: HIP runtime error";
  }
  return "NVFP4: unknown status";
}

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols) { return quant_ws(1, rows, cols, true); }

nvfp4_status nvfp4_quantize(const void *x, nvfp4_dtype x_type, int64_t rows, int64_t cols,
                            int64_t ld_x, uint8_t *q, uint8_t *s, float *g, int static_global,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(x_type) || !quant_shape_ok(rows, cols) || ld_x < cols || !g)
    return NVFP4_ERR_INVALID_ARG;
  if (rows > 0 && (!x || !q || !s)) return NVFP4_ERR_INVALID_ARG;
  if (rows > 0 && ld_x > kI32Max * 64ll) return NVFP4_ERR_INVALID_ARG;
  if (!static_global) {
    const size_t need = quant_ws(1, rows, cols, true);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
      return NVFP4_ERR_INVALID_ARG;
  } else if (rows == 0) {
    return NVFP4_OK;
  }
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  return quantize_impl(x, x_type, rows, cols, ld_x, q, s, g, static_global, workspace, stream);
}

nvfp4_status nvfp4_quantize_noalloc(const void *x, nvfp4_dtype x_type, int64_t rows, int64_t cols,
                                    int64_t ld_x, uint8_t *q, uint8_t *s, float *g, int static_global,
                                    hipStream_t stream) {
  if (!valid_dtype(x_type) || !quant_shape_ok(rows, cols) || ld_x < cols || !g)
    return NVFP4_ERR_INVALID_ARG;
  if (rows > 0 && (!x || !q || !s)) return NVFP4_ERR_INVALID_ARG;
  if (rows > 0 && ld_x > kI32Max * 64ll) return NVFP4_ERR_INVALID_ARG;
  if (quant_ws(1, rows, cols, true) > kScratchBytes) return NVFP4_ERR_INVALID_ARG;
  if (static_global && rows == 0) return NVFP4_OK;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  void *ws = nullptr;
  if (!static_global && (st = device_scratch(&ws, stream)) != NVFP4_OK) return st;
  return quantize_impl(x, x_type, rows, cols, ld_x, q, s, g, static_global, ws, stream);
}

size_t nvfp4_quantize_batched_workspace_size(int64_t batch, int64_t rows, int64_t cols) {
  return quant_ws(batch, rows, cols, false);
}

nvfp4_status nvfp4_quantize_batched(const void *x, nvfp4_dtype x_type, int64_t batch,
                                    int64_t rows, int64_t cols, uint8_t *q, uint8_t *s, float *g,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(x_type) || !quant_shape_ok(rows, cols) || batch < 0 || batch > 65535)
    return NVFP4_ERR_INVALID_ARG;
  if (batch == 0) return NVFP4_OK;
  if (!g || (rows > 0 && (!x || !q || !s))) return NVFP4_ERR_INVALID_ARG;
  const size_t need = quant_ws(batch, rows, cols, false);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 3u))
    return NVFP4_ERR_INVALID_ARG;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  const bool vec = aligned16(x) && (cols * (int64_t)dtype_size(x_type)) % 16 == 0;
  QuantParams p = make_quant(x, rows, cols, cols, q, s, g, workspace, 0);
  return from_hip(launch_quantize(p, x_type == NVFP4_BF16, vec, (uint32_t)batch, nullptr, stream));
}

nvfp4_status nvfp4_qdq(const void *x, nvfp4_dtype x_type, int64_t rows, int64_t cols,
                       int64_t ld_x, void *y, int64_t ld_y, float *g, int static_global,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(x_type) || !quant_shape_ok(rows, cols) || ld_x < cols || ld_y < cols || !g)
    return NVFP4_ERR_INVALID_ARG;
  if (rows > 0 && (!x || !y)) return NVFP4_ERR_INVALID_ARG;
  if (rows > 0 && (ld_x > kI32Max * 64ll || ld_y > kI32Max * 64ll)) return NVFP4_ERR_INVALID_ARG;
  if (x && y && x == y && ld_x != ld_y) return NVFP4_ERR_INVALID_ARG;
  if (!static_global) {
    const size_t need = quant_ws(1, rows, cols, true);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
      return NVFP4_ERR_INVALID_ARG;
  } else if (rows == 0) {
    return NVFP4_OK;
  }
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  const int64_t es = (int64_t)dtype_size(x_type);
  const bool vec = aligned16(x) && aligned16(y) && (ld_x * es) % 16 == 0 && (ld_y * es) % 16 == 0;
  ResidentState *rs = static_cast<ResidentState *>(workspace);
  void *partials = workspace ? static_cast<uint8_t *>(workspace) + kResidentStateBytes : nullptr;
  QuantParams p = make_quant(x, rows, cols, ld_x, nullptr, nullptr, g, partials, static_global ? 1 : 0);
  p.y = y;
  p.ld_y = ld_y;
  return from_hip(launch_quantize(p, x_type == NVFP4_BF16, vec, 1, rs, stream));
}

nvfp4_status nvfp4_quantize_4over6(const void *x, nvfp4_dtype x_type, int64_t batch,
                                   int64_t rows, int64_t cols, uint8_t *q, uint8_t *s, float *g,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(x_type) || !quant_shape_ok(rows, cols) || batch < 0 || batch > 65535)
    return NVFP4_ERR_INVALID_ARG;
  if (batch == 0) return NVFP4_OK;
  if (!g || (rows > 0 && (!x || !q || !s))) return NVFP4_ERR_INVALID_ARG;
  const size_t need = quant_ws(batch, rows, cols, false);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 3u))
    return NVFP4_ERR_INVALID_ARG;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  const bool vec = aligned16(x) && (cols * (int64_t)dtype_size(x_type)) % 16 == 0;
  QuantParams p = make_quant(x, rows, cols, cols, q, s, g, workspace, 0);
  p.four6 = 1;
  return from_hip(launch_quantize(p, x_type == NVFP4_BF16, vec, (uint32_t)batch, nullptr, stream));
}

nvfp4_status nvfp4_gemm(const uint8_t *a_q, const uint8_t *a_s, const float *a_g,
                        const uint8_t *b_q, const uint8_t *b_s, const float *b_g, int64_t M,
                        int64_t N, int64_t K, void *c, nvfp4_dtype c_type, int64_t ldc,
                        hipStream_t stream) {
  if (!valid_dtype(c_type) || M < 0 || N < 0 || K <= 0 || K % 16 != 0 || ldc < N)
    return NVFP4_ERR_INVALID_ARG;
  if (M > kI32Max || N > kI32Max || K > kI32Max) return NVFP4_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_q || !a_s || !a_g || !b_q || !b_s || !b_g || !c) return NVFP4_ERR_INVALID_ARG;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  GemmParams p{};
  p.a_q = a_q; p.a_s = a_s; p.a_g = a_g;
  p.b_q = b_q; p.b_s = b_s; p.b_g = b_g;
  p.M = (uint32_t)M; p.N = (uint32_t)N; p.K = (uint32_t)K;
  p.c = c; p.ldc = ldc;
  return from_hip(launch_gemm(p, c_type == NVFP4_BF16 ? OutType::BF16 : OutType::F32, stream));
}

size_t nvfp4_fp8_quantize_workspace_size(int64_t rows, int64_t cols) { return quant_ws(1, rows, cols, true); }

nvfp4_status nvfp4_fp8_quantize(const void *x, nvfp4_dtype x_type, int64_t rows, int64_t cols,
                                int64_t ld_x, uint8_t *q, float *g, int static_scale, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(x_type) || !quant_shape_ok(rows, cols) || ld_x < cols || !g)
    return NVFP4_ERR_INVALID_ARG;
  if (rows > 0 && (!x || !q || !aligned16(q))) return NVFP4_ERR_INVALID_ARG;
  if (rows > 0 && ld_x > kI32Max * 64ll) return NVFP4_ERR_INVALID_ARG;
  if (!static_scale) {
    const size_t need = quant_ws(1, rows, cols, true);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
      return NVFP4_ERR_INVALID_ARG;
  } else if (rows == 0) {
    return NVFP4_OK;
  }
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  const bool vec = aligned16(x) && (ld_x * (int64_t)dtype_size(x_type)) % 16 == 0;
  ResidentState *rs = static_cast<ResidentState *>(workspace);
  void *partials = workspace ? static_cast<uint8_t *>(workspace) + kResidentStateBytes : nullptr;
  QuantParams p = make_quant(x, rows, cols, ld_x, q, nullptr, g, partials, static_scale ? 1 : 0);
  p.fp8 = 1;
  return from_hip(launch_quantize(p, x_type == NVFP4_BF16, vec, 1, rs, stream));
}

nvfp4_status nvfp4_fp8_gemm(const uint8_t *a_q, const float *a_g, const uint8_t *b_q,
                            const float *b_g, int64_t M, int64_t N, int64_t K, void *c,
                            nvfp4_dtype c_type, int64_t ldc, hipStream_t stream) {
  if (!valid_dtype(c_type) || M < 0 || N < 0 || K <= 0 || K % 16 != 0 || ldc < N)
    return NVFP4_ERR_INVALID_ARG;
  if (M > kI32Max || N > kI32Max || K > kI32Max) return NVFP4_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_q || !a_g || !b_q || !b_g || !c || !aligned16(a_q) || !aligned16(b_q))
    return NVFP4_ERR_INVALID_ARG;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  Fp8GemmParams p{};
  p.a_q = a_q; p.a_g = a_g;
  p.b_q = b_q; p.b_g = b_g;
  p.M = (uint32_t)M; p.N = (uint32_t)N; p.K = (uint32_t)K;
  p.c = c; p.ldc = ldc;
  return from_hip(launch_fp8_gemm(p, c_type == NVFP4_BF16 ? OutType::BF16 : OutType::F32, stream));
}

size_t nvfp4_moe_route_workspace_size(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E <= 0) return 0;
  return round_up(route_workspace_bytes(T, E, k), 256);
}

nvfp4_status nvfp4_moe_route(const float *logits, int64_t T, int32_t E, int32_t k,
                             int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                             int32_t *src_row, int32_t *inv, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E) return NVFP4_ERR_INVALID_ARG;
  if (T * (int64_t)k > kI32Max || (T + 63) / 64 * (int64_t)E > kI32Max) return NVFP4_ERR_INVALID_ARG;
  if (!expert_offsets) return NVFP4_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !src_row || !inv)) return NVFP4_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < nvfp4_moe_route_workspace_size(T, E, k) ||
      ((uintptr_t)workspace & 3u))
    return NVFP4_ERR_INVALID_ARG;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  return from_hip(launch_route(logits, T, E, k, topk_ids, topk_w, expert_offsets, src_row, inv,
                               workspace, stream));
}

nvfp4_status nvfp4_moe_grouped_gemm(const uint8_t *a_q, const uint8_t *a_s, const float *a_g,
                                    int64_t a_rows, const int32_t *src_row,
                                    const int32_t *expert_offsets, int32_t E, int64_t R,
                                    const uint8_t *w_q, const uint8_t *w_s, const float *w_g,
                                    int64_t N, int64_t K, void *c, nvfp4_dtype c_type,
                                    nvfp4_epilogue epilogue, hipStream_t stream) {
  if (!valid_dtype(c_type) || E < 1 || R < 0 || N <= 0 || K <= 0 || K % 16 != 0 || a_rows < 0)
    return NVFP4_ERR_INVALID_ARG;
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_SILU_GATE) return NVFP4_ERR_INVALID_ARG;
  if (epilogue == NVFP4_EPI_SILU_GATE && N % 2 != 0) return NVFP4_ERR_INVALID_ARG;
  if (R > kI32Max || N > kI32Max || K > kI32Max || a_rows > kI32Max || E > 65536)
    return NVFP4_ERR_INVALID_ARG;
  if (R == 0) return NVFP4_OK;
  if (!a_q || !a_s || !a_g || !expert_offsets || !w_q || !w_s || !w_g || !c || a_rows == 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!src_row && a_rows < R) return NVFP4_ERR_INVALID_ARG;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  GemmParams p{};
  p.a_q = a_q; p.a_s = a_s; p.a_g = a_g;
  p.b_q = w_q; p.b_s = w_s; p.b_g = w_g;
  p.M = (uint32_t)R; p.N = (uint32_t)N; p.K = (uint32_t)K;
  p.c = c;
  p.ldc = epilogue == NVFP4_EPI_SILU_GATE ? N / 2 : N;
  p.a_rows = (uint32_t)a_rows;
  p.src_row = src_row;
  p.expert_offsets = expert_offsets;
  p.E = (uint32_t)E;
  p.b_mstride_q = N * (K / 2);
  p.b_mstride_s = N * (K / 16);
  return from_hip(launch_grouped_gemm(
      p, (uint32_t)R, c_type == NVFP4_BF16 ? OutType::BF16 : OutType::F32,
      epilogue == NVFP4_EPI_SILU_GATE ? Epilogue::SiluGate : Epilogue::None, stream));
}

nvfp4_status nvfp4_moe_grouped_gemm_silu_nvfp4(
    const uint8_t *a_q, const uint8_t *a_s, const float *a_g, int64_t a_rows,
    const int32_t *src_row, const int32_t *expert_offsets, int32_t E, int64_t R,
    const uint8_t *w_q, const uint8_t *w_s, const float *w_g, int64_t N, int64_t K, uint8_t *h_q,
    uint8_t *h_s, const float *h_g, hipStream_t stream) {
  if (E < 1 || R < 0 || N <= 0 || K <= 0 || K % 16 != 0 || a_rows < 0 || N % 32 != 0)
    return NVFP4_ERR_INVALID_ARG;
  if (R > kI32Max || N > kI32Max || K > kI32Max || a_rows > kI32Max || E > 65536)
    return NVFP4_ERR_INVALID_ARG;
  if (R == 0) return NVFP4_OK;
  if (!a_q || !a_s || !a_g || !expert_offsets || !w_q || !w_s || !w_g || !h_q || !h_s || !h_g ||
      a_rows == 0)
    return NVFP4_ERR_INVALID_ARG;
  if (!src_row && a_rows < R) return NVFP4_ERR_INVALID_ARG;
  GemmParams p{};
  p.a_q = a_q; p.a_s = a_s; p.a_g = a_g;
  p.b_q = w_q; p.b_s = w_s; p.b_g = w_g;
  p.M = (uint32_t)R; p.N = (uint32_t)N; p.K = (uint32_t)K;
  p.c = nullptr;
  p.ldc = N / 2;
  p.a_rows = (uint32_t)a_rows;
  p.src_row = src_row;
  p.expert_offsets = expert_offsets;
  p.E = (uint32_t)E;
  p.b_mstride_q = N * (K / 2);
  p.b_mstride_s = N * (K / 16);
  p.h_q = h_q; p.h_s = h_s; p.h_g = h_g;
  if (!grouped_nvfp4_out_supported(p)) return NVFP4_ERR_UNSUPPORTED;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  return from_hip(launch_grouped_gemm(p, (uint32_t)R, OutType::F32, Epilogue::SiluGateNvfp4, stream));
}

nvfp4_status nvfp4_moe_combine(const void *y, nvfp4_dtype y_type, const float *topk_w,
                               const int32_t *inv, int64_t T, int32_t k, int64_t H, int64_t R,
                               void *out, nvfp4_dtype out_type, hipStream_t stream) {
  if (!valid_dtype(y_type) || !valid_dtype(out_type) || T < 0 || k < 1 || k > 32 || H <= 0 ||
      R < 0 || T * (int64_t)k > R || H > kI32Max || T > kI32Max)
    return NVFP4_ERR_INVALID_ARG;
  if (T == 0) return NVFP4_OK;
  if (!y || !topk_w || !inv || !out) return NVFP4_ERR_INVALID_ARG;
  nvfp4_status st = check_device();
  if (st != NVFP4_OK) return st;
  return from_hip(launch_combine(y, y_type == NVFP4_BF16, topk_w, inv, T, k, H, out,
                                 out_type == NVFP4_BF16, stream));
}

}  // extern "C"
