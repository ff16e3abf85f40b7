// C ABI of the NVFP4 W4A4 layer: argument validation and kernel launches.
// Every entry point validates all arguments before touching the device; on an
// error nothing is enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/nvfp4_w4a4.h"
#include "kernels.h"

namespace {

using nvfp4::kWorkspaceBytes;

constexpr int64_t kMaxDim = int64_t(1) << 31;        // kernel index range

bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

std::atomic<int> g_path_flags{0};

// Cached per-device check that the current device is gfx950.  The cache only
// memoises hipGetDeviceProperties; the NVFP4_PATH_REJECT_DEVICE flag makes
// every device fail the check (it never makes another device pass).
nvfp4_status_t check_device() {
  static std::atomic<int> cache[64];
  if (g_path_flags.load(std::memory_order_relaxed) & nvfp4::kPathRejectDevice)
    return NVFP4_ERR_UNSUPPORTED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return NVFP4_ERR_UNSUPPORTED;
  }
  if (dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) return c == 1 ? NVFP4_OK : NVFP4_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return NVFP4_ERR_UNSUPPORTED;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? NVFP4_OK : NVFP4_ERR_UNSUPPORTED;
}

nvfp4_status_t launched(hipError_t e) {
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

// Workspace of nvfp4_quantize_act_noalloc: a fixed 15 616 bytes (amax
// partials, alpha's parameters and the two decision tables), the same for
// every tensor size.  Each device holds its own copy of this array from the
// module's load until the process ends; all calls on a device share it.
static __device__ __align__(256) uint8_t scratch[kWorkspaceBytes];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.  The array's name is a host
// stand-in in host code; only this address may be passed to kernels.
nvfp4_status_t scratch_address(void** out) {
  static std::atomic<void*> addr[64];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return NVFP4_ERR_UNSUPPORTED;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return NVFP4_ERR_LAUNCH;
      }
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return NVFP4_OK;
}

// Common validation of a BF16 source [rows][K] with the given strides.
nvfp4_status_t check_source(const void* x, int64_t rows, int64_t K,
                            int64_t stride_row, int64_t stride_k) {
  if (rows < 0 || K <= 0 || K % 16 != 0 || rows >= kMaxDim || K >= kMaxDim)
    return NVFP4_ERR_SHAPE;
  if (rows * (K / 16) >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (stride_k == 1) {
    if (stride_row < K) return NVFP4_ERR_SHAPE;
    if (rows > 0 && (!aligned(x, 16) || stride_row % 8 != 0)) return NVFP4_ERR_ALIGN;
  } else {
    if (stride_row < 1 || stride_k < 1) return NVFP4_ERR_SHAPE;
    if (rows > 0 && !aligned(x, 2)) return NVFP4_ERR_ALIGN;
  }
  return NVFP4_OK;
}

nvfp4_status_t check_outputs(const void* y_f32, const void* y_bf16, int64_t N,
                             int64_t ld_y) {
  if (y_f32 == nullptr && y_bf16 == nullptr) return NVFP4_ERR_NULL;
  if (ld_y < N) return NVFP4_ERR_SHAPE;
  if (y_f32 != nullptr && !aligned(y_f32, 4)) return NVFP4_ERR_ALIGN;
  if (y_bf16 != nullptr && !aligned(y_bf16, 2)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

// use_scratch: the workspace is the device's `scratch` array (ws ignored).
nvfp4_status_t quantize_common(const void* x, int64_t rows, int64_t K,
                               int64_t stride_row, int64_t stride_k,
                               const float* alpha_in, float* alpha_out,
                               uint8_t* codes, uint8_t* scales, void* ws,
                               size_t ws_bytes, hipStream_t stream,
                               bool use_scratch = false) {
  if (alpha_out == nullptr) return NVFP4_ERR_NULL;
  if (rows > 0 && (x == nullptr || codes == nullptr || scales == nullptr))
    return NVFP4_ERR_NULL;
  nvfp4_status_t st = check_source(x, rows, K, stride_row, stride_k);
  if (st != NVFP4_OK) return st;
  if (!use_scratch) {
    if (ws == nullptr || ws_bytes < kWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
  }
  if (rows > 0 && !aligned(codes, 8)) return NVFP4_ERR_ALIGN;
  if ((st = check_device()) != NVFP4_OK) return st;
  if (use_scratch && (st = scratch_address(&ws)) != NVFP4_OK) return st;

  uint8_t* w = static_cast<uint8_t*>(ws);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  int n_partials = 0;
  if (alpha_in == nullptr && rows > 0) {
    if (nvfp4::launch_amax(xs, rows, K, stride_row, stride_k, w, &n_partials, stream) != hipSuccess)
      return NVFP4_ERR_LAUNCH;
  }
  if (nvfp4::launch_prepare(w + nvfp4::kWsPartials, n_partials, alpha_in, alpha_out, w, stream) !=
      hipSuccess)
    return NVFP4_ERR_LAUNCH;
  if (rows == 0) return NVFP4_OK;
  return launched(nvfp4::launch_quantize(xs, rows, K, stride_row, stride_k, w, codes, scales,
                                         stream));
}

}  // namespace

int nvfp4::path_flags() { return g_path_flags.load(std::memory_order_relaxed); }

extern "C" {

void nvfp4_set_path_flags(int flags) {
  g_path_flags.store(flags & (nvfp4::kPathGemmGrid | nvfp4::kPathDecodeDirect |
                              nvfp4::kPathRejectDevice),
                     std::memory_order_relaxed);
}

int nvfp4_path_flags(void) { return g_path_flags.load(std::memory_order_relaxed); }

const char* nvfp4_status_string(nvfp4_status_t s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid size, stride or group offsets (K must be a positive multiple of 16)";
    case NVFP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case NVFP4_ERR_UNSUPPORTED: return "the current HIP device is not gfx950 (MI355X)";
    case NVFP4_ERR_LAUNCH: return "a HIP kernel launch failed";
    case NVFP4_ERR_WORKSPACE: return "workspace is NULL or smaller than nvfp4_workspace_bytes()";
  }
  return "unknown status";
}

size_t nvfp4_workspace_bytes(void) { return kWorkspaceBytes; }

nvfp4_status_t nvfp4_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ld_x,
                                  const float* alpha_in, float* alpha_out, uint8_t* codes,
                                  uint8_t* scales, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  return quantize_common(x_bf16, M, K, ld_x, 1, alpha_in, alpha_out, codes, scales, workspace,
                         workspace_bytes, stream);
}

nvfp4_status_t nvfp4_quantize_act_noalloc(const void* x_bf16, int64_t M, int64_t K,
                                          int64_t ld_x, const float* alpha_in,
                                          float* alpha_out, uint8_t* codes, uint8_t* scales,
                                          hipStream_t stream) {
  return quantize_common(x_bf16, M, K, ld_x, 1, alpha_in, alpha_out, codes, scales, nullptr, 0,
                         stream, true);
}

size_t nvfp4_rmsnorm_workspace_bytes(int64_t M) {
  if (M < 0) return 0;
  return nvfp4::kWsRowR + 4 * (size_t)M;
}

nvfp4_status_t nvfp4_rmsnorm_quantize_act(const void* x_bf16, const void* gamma_bf16, int64_t M,
                                          int64_t K, int64_t ld_x, float eps,
                                          const float* alpha_in, float* alpha_out,
                                          uint8_t* codes, uint8_t* scales, uint16_t* y_bf16,
                                          int64_t ld_y, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  if (alpha_out == nullptr) return NVFP4_ERR_NULL;
  if (M > 0 && (x_bf16 == nullptr || gamma_bf16 == nullptr || codes == nullptr ||
                scales == nullptr))
    return NVFP4_ERR_NULL;
  if (K > nvfp4::kRmsMaxK || !(eps >= 0.0f) || eps > 3.0e38f) return NVFP4_ERR_SHAPE;
  nvfp4_status_t st = check_source(x_bf16, M, K, ld_x, 1);
  if (st != NVFP4_OK) return st;
  if (M > 0 && !aligned(gamma_bf16, 16)) return NVFP4_ERR_ALIGN;
  if (y_bf16 != nullptr && M > 0) {
    if (ld_y < K) return NVFP4_ERR_SHAPE;
    if (!aligned(y_bf16, 16) || ld_y % 8 != 0) return NVFP4_ERR_ALIGN;
  }
  if (workspace == nullptr || workspace_bytes < kWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  if (M > 0 && !aligned(codes, 8)) return NVFP4_ERR_ALIGN;
  if ((st = check_device()) != NVFP4_OK) return st;

  uint8_t* w = static_cast<uint8_t*>(workspace);
  nvfp4::RmsQuantArgs a;
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.gamma = static_cast<const uint16_t*>(gamma_bf16);
  a.M = M;
  a.K = K;
  a.ld_x = ld_x;
  a.eps = eps;
  a.ws = w;
  a.codes = codes;
  a.scales = scales;
  a.y_out = y_bf16;
  a.ld_y = ld_y;
  // room for each row's r: the amax pass keeps it for the quantise pass
  a.row_r = (alpha_in == nullptr && workspace_bytes >= nvfp4_rmsnorm_workspace_bytes(M))
                ? reinterpret_cast<float*>(w + nvfp4::kWsRowR)
                : nullptr;
  int n_partials = 0;
  if (alpha_in == nullptr && M > 0) {
    a.amax_pass = true;
    if (nvfp4::launch_rmsnorm_quant(a, stream) != hipSuccess) return NVFP4_ERR_LAUNCH;
    n_partials = nvfp4::rmsnorm_amax_grid(M, K);
  }
  if (nvfp4::launch_prepare(w + nvfp4::kWsPartials, n_partials, alpha_in, alpha_out, w, stream) !=
      hipSuccess)
    return NVFP4_ERR_LAUNCH;
  a.amax_pass = false;
  return launched(nvfp4::launch_rmsnorm_quant(a, stream));
}

nvfp4_status_t nvfp4_quantize_weights(const void* w_bf16, int64_t N, int64_t K,
                                      int64_t stride_n, int64_t stride_k, float* alpha_out,
                                      uint8_t* codes, uint8_t* scales, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (stride_k != 1 && stride_n != 1) return NVFP4_ERR_SHAPE;
  return quantize_common(w_bf16, N, K, stride_n, stride_k, nullptr, alpha_out, codes, scales,
                         workspace, workspace_bytes, stream);
}

nvfp4_status_t nvfp4_tensor_alpha(const void* x_bf16, int64_t M, int64_t K, int64_t ld_x,
                                  float* alpha_out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (alpha_out == nullptr || (M > 0 && x_bf16 == nullptr)) return NVFP4_ERR_NULL;
  nvfp4_status_t st = check_source(x_bf16, M, K, ld_x, 1);
  if (st != NVFP4_OK) return st;
  if (workspace == nullptr || workspace_bytes < kWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  if ((st = check_device()) != NVFP4_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(workspace);
  int n_partials = 0;
  if (M > 0 &&
      nvfp4::launch_amax(static_cast<const uint16_t*>(x_bf16), M, K, ld_x, 1, w, &n_partials,
                         stream) != hipSuccess)
    return NVFP4_ERR_LAUNCH;
  return launched(nvfp4::launch_prepare(w + nvfp4::kWsPartials, n_partials, nullptr, alpha_out, w,
                                        stream));
}

static nvfp4_status_t gemm_common(const uint8_t* a_codes, const uint8_t* a_scales,
                                  const float* alpha_a, int64_t a_rows,
                                  const int32_t* a_row_index, const uint8_t* b_codes,
                                  const uint8_t* b_scales, const float* alpha_b,
                                  const float* alpha_b_rows, int64_t M,
                                  int64_t N, int64_t K, int32_t num_groups,
                                  const int64_t* group_offsets, float* y_f32, uint16_t* y_bf16,
                                  int64_t ld_y, hipStream_t stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || M >= kMaxDim || N >= kMaxDim ||
      K >= kMaxDim || a_rows < 0 || num_groups < 1)
    return NVFP4_ERR_SHAPE;
  if (num_groups > 1 && group_offsets == nullptr) return NVFP4_ERR_NULL;
  nvfp4_status_t st = check_outputs(y_f32, y_bf16, N, ld_y);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !alpha_a || !b_codes || !b_scales || !(alpha_b || alpha_b_rows))
    return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16)) return NVFP4_ERR_ALIGN;
  if (K % 128 == 0 && (!aligned(a_scales, 8) || !aligned(b_scales, 8))) return NVFP4_ERR_ALIGN;
  if (a_row_index == nullptr && a_rows < M) return NVFP4_ERR_SHAPE;
  // the kernels address each operand with 32-bit byte offsets
  constexpr int64_t kMaxBytes = (int64_t(1) << 32) - 1;
  if ((a_row_index ? a_rows : M) * (K / 2) > kMaxBytes || N * (K / 2) > kMaxBytes)
    return NVFP4_ERR_SHAPE;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::W4A4Args a;
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.alpha_a = alpha_a;
  a.a_row_index = a_row_index;
  a.b_codes = b_codes;
  a.b_scales = b_scales;
  a.alpha_b = alpha_b;
  a.alpha_b_rows = alpha_b_rows;
  a.M = M;
  a.N = N;
  a.K = K;
  a.num_groups = num_groups;
  a.group_offsets = group_offsets;
  a.y_f32 = y_f32;
  a.y_bf16 = y_bf16;
  a.ld_y = ld_y;
  a.a_bf16 = nullptr;
  a.ld_a = 0;
  a.ws = nullptr;
  a.h_bf16 = nullptr;
  a.ld_h = 0;
  a.h_partials = nullptr;
  return launched(nvfp4::launch_w4a4(a, stream));
}

nvfp4_status_t w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* alpha_a,
                         const uint8_t* b_codes, const uint8_t* b_scales, const float* alpha_b,
                         int64_t M, int64_t N, int64_t K, float* y_f32, uint16_t* y_bf16,
                         int64_t ld_y, hipStream_t stream) {
  return gemm_common(a_codes, a_scales, alpha_a, M, nullptr, b_codes, b_scales, alpha_b, nullptr,
                     M, N, K, 1, nullptr, y_f32, y_bf16, ld_y, stream);
}

nvfp4_status_t w4a4_gemm_multi(const uint8_t* a_codes, const uint8_t* a_scales,
                               const float* alpha_a, const uint8_t* b_codes,
                               const uint8_t* b_scales, const float* alpha_b_rows, int64_t M,
                               int64_t N, int64_t K, float* y_f32, uint16_t* y_bf16,
                               int64_t ld_y, hipStream_t stream) {
  if (alpha_b_rows == nullptr) return NVFP4_ERR_NULL;
  return gemm_common(a_codes, a_scales, alpha_a, M, nullptr, b_codes, b_scales, nullptr,
                     alpha_b_rows, M, N, K, 1, nullptr, y_f32, y_bf16, ld_y, stream);
}

size_t w4a4_gemm_silu_mul_workspace_bytes(int64_t M, int64_t N) {
  if (M < 0 || N < 0) return 0;
  return kWorkspaceBytes + 4 * (size_t)nvfp4::w4a4_silu_tiles_max(M, N);
}

nvfp4_status_t w4a4_gemm_silu_mul_quantize(const uint8_t* a_codes, const uint8_t* a_scales,
                                           const float* alpha_a, const uint8_t* b_codes,
                                           const uint8_t* b_scales, const float* alpha_b_rows,
                                           int64_t M, int64_t N, int64_t K, uint16_t* h_bf16,
                                           int64_t ld_h, float* alpha_h_out, uint8_t* h_codes,
                                           uint8_t* h_scales, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || N % 64 != 0 || M >= kMaxDim || N >= kMaxDim ||
      K >= kMaxDim)
    return NVFP4_ERR_SHAPE;
  if (alpha_h_out == nullptr) return NVFP4_ERR_NULL;
  const int64_t nh = N / 2;
  if (M > 0 && N > 0) {
    if (!a_codes || !a_scales || !alpha_a || !b_codes || !b_scales || !alpha_b_rows || !h_bf16 ||
        !h_codes || !h_scales)
      return NVFP4_ERR_NULL;
    if (ld_h < nh) return NVFP4_ERR_SHAPE;
    if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(h_bf16, 16) || ld_h % 8 != 0)
      return NVFP4_ERR_ALIGN;
    if (K % 128 == 0 && (!aligned(a_scales, 8) || !aligned(b_scales, 8))) return NVFP4_ERR_ALIGN;
    if (!aligned(h_codes, 8)) return NVFP4_ERR_ALIGN;
    constexpr int64_t kMaxBytes = (int64_t(1) << 32) - 1;
    if (M * (K / 2) > kMaxBytes || N * (K / 2) > kMaxBytes) return NVFP4_ERR_SHAPE;
    if (M * (nh / 16) >= kMaxDim) return NVFP4_ERR_SHAPE;     // H's blocks, as the quantiser's
  }
  if (workspace == nullptr || workspace_bytes < w4a4_gemm_silu_mul_workspace_bytes(M, N))
    return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  nvfp4_status_t st = check_device();
  if (st != NVFP4_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(workspace);
  uint32_t* partials = reinterpret_cast<uint32_t*>(w + kWorkspaceBytes);
  int n_partials = 0;
  if (M > 0 && N > 0) {
    nvfp4::W4A4Args a;
    a.a_codes = a_codes;
    a.a_scales = a_scales;
    a.alpha_a = alpha_a;
    a.a_row_index = nullptr;
    a.b_codes = b_codes;
    a.b_scales = b_scales;
    a.alpha_b = nullptr;
    a.alpha_b_rows = alpha_b_rows;
    a.M = M;
    a.N = N;
    a.K = K;
    a.num_groups = 1;
    a.group_offsets = nullptr;
    a.y_f32 = nullptr;
    a.y_bf16 = nullptr;
    a.ld_y = 0;
    a.a_bf16 = nullptr;
    a.ld_a = 0;
    a.ws = nullptr;
    a.h_bf16 = h_bf16;
    a.ld_h = ld_h;
    a.h_partials = partials;
    if (nvfp4::launch_w4a4_silu(a, stream) != hipSuccess) return NVFP4_ERR_LAUNCH;
    n_partials = (int)nvfp4::w4a4_tiles(M, N);
  }
  // alpha of H from the tiles' maxima, then H's codes and scales
  if (nvfp4::launch_prepare(reinterpret_cast<const uint8_t*>(partials), n_partials, nullptr,
                            alpha_h_out, w, stream) != hipSuccess)
    return NVFP4_ERR_LAUNCH;
  if (M == 0 || N == 0) return NVFP4_OK;
  return launched(nvfp4::launch_quantize(h_bf16, M, nh, ld_h, 1, w, h_codes, h_scales, stream));
}

nvfp4_status_t w4a4_gemm_decode(const uint8_t* a_codes, const uint8_t* a_scales,
                                const float* alpha_a, const uint8_t* b_codes,
                                const uint8_t* b_scales, const float* alpha_b,
                                const float* alpha_b_rows, int64_t M, int64_t N, int64_t K,
                                float* y_f32, uint16_t* y_bf16, int64_t ld_y,
                                hipStream_t stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || M > NVFP4_DECODE_MAX_ROWS || N >= kMaxDim ||
      K >= kMaxDim)
    return NVFP4_ERR_SHAPE;
  nvfp4_status_t st = check_outputs(y_f32, y_bf16, N, ld_y);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !alpha_a || !b_codes || !b_scales || !(alpha_b || alpha_b_rows))
    return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16)) return NVFP4_ERR_ALIGN;
  if (K % 32 == 0 && (!aligned(a_scales, 2) || !aligned(b_scales, 2))) return NVFP4_ERR_ALIGN;
  // the kernel addresses each operand with 32-bit byte offsets
  if (N * (K / 2) > (int64_t(1) << 32) - 1) return NVFP4_ERR_SHAPE;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::DecodeArgs a;
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.alpha_a = alpha_a;
  a.b_codes = b_codes;
  a.b_scales = b_scales;
  a.alpha_b = alpha_b;
  a.alpha_b_rows = alpha_b_rows;
  a.M = M;
  a.N = N;
  a.K = K;
  a.y_f32 = y_f32;
  a.y_bf16 = y_bf16;
  a.ld_y = ld_y;
  return launched(nvfp4::launch_w4a4_decode(a, stream));
}

nvfp4_status_t w4a4_gemm_grouped(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const float* alpha_a, int64_t a_rows,
                                 const int32_t* a_row_index, const uint8_t* b_codes,
                                 const uint8_t* b_scales, const float* alpha_b, int64_t M,
                                 int64_t N, int64_t K, int32_t num_groups,
                                 const int64_t* group_offsets, float* y_f32, uint16_t* y_bf16,
                                 int64_t ld_y, hipStream_t stream) {
  if (group_offsets == nullptr) return NVFP4_ERR_NULL;
  if (alpha_b == nullptr) return NVFP4_ERR_NULL;
  return gemm_common(a_codes, a_scales, alpha_a, a_rows, a_row_index, b_codes, b_scales,
                     alpha_b, nullptr, M, N, K, num_groups, group_offsets, y_f32, y_bf16, ld_y,
                     stream);
}

nvfp4_status_t w4a4_gemm_fused_act(const void* x_bf16, int64_t ld_x, const float* alpha_a,
                                   const uint8_t* b_codes, const uint8_t* b_scales,
                                   const float* alpha_b, int64_t M, int64_t N, int64_t K,
                                   float* y_f32, uint16_t* y_bf16, int64_t ld_y,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || M >= kMaxDim || N >= kMaxDim)
    return NVFP4_ERR_SHAPE;
  nvfp4_status_t st = check_outputs(y_f32, y_bf16, N, ld_y);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!x_bf16 || !alpha_a || !b_codes || !b_scales || !alpha_b) return NVFP4_ERR_NULL;
  if ((st = check_source(x_bf16, M, K, ld_x, 1)) != NVFP4_OK) return st;
  if (!aligned(b_codes, 16)) return NVFP4_ERR_ALIGN;
  if (K % 128 == 0 && !aligned(b_scales, 8)) return NVFP4_ERR_ALIGN;
  // the kernel addresses the weight with 32-bit byte offsets
  if (N * (K / 2) > (int64_t(1) << 32) - 1) return NVFP4_ERR_SHAPE;
  if (workspace == nullptr || workspace_bytes < kWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  if ((st = check_device()) != NVFP4_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(workspace);
  // decision tables for alpha_a, then the GEMM quantises its A tiles with them
  float* alpha_slot = reinterpret_cast<float*>(w + nvfp4::kWsParams + sizeof(nvfp4::QuantParams));
  if (nvfp4::launch_prepare(w, 0, alpha_a, alpha_slot, w, stream) != hipSuccess)
    return NVFP4_ERR_LAUNCH;
  nvfp4::W4A4Args a;
  a.a_codes = nullptr;
  a.a_scales = nullptr;
  a.alpha_a = alpha_a;
  a.a_row_index = nullptr;
  a.b_codes = b_codes;
  a.b_scales = b_scales;
  a.alpha_b = alpha_b;
  a.alpha_b_rows = nullptr;
  a.M = M;
  a.N = N;
  a.K = K;
  a.num_groups = 1;
  a.group_offsets = nullptr;
  a.y_f32 = y_f32;
  a.y_bf16 = y_bf16;
  a.ld_y = ld_y;
  a.a_bf16 = static_cast<const uint16_t*>(x_bf16);
  a.ld_a = ld_x;
  a.ws = w;
  a.h_bf16 = nullptr;
  a.ld_h = 0;
  a.h_partials = nullptr;
  return launched(nvfp4::launch_w4a4_fused(a, stream));
}

nvfp4_status_t bf16_gemm_baseline(const void* x_bf16, const void* w_bf16, int64_t M, int64_t N,
                                  int64_t K, int32_t num_groups, const int64_t* group_offsets,
                                  float* y_f32, uint16_t* y_bf16, int64_t ld_y,
                                  hipStream_t stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || M >= kMaxDim || N >= kMaxDim ||
      K >= kMaxDim || num_groups < 1)
    return NVFP4_ERR_SHAPE;
  if (num_groups > 1 && group_offsets == nullptr) return NVFP4_ERR_NULL;
  nvfp4_status_t st = check_outputs(y_f32, y_bf16, N, ld_y);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!x_bf16 || !w_bf16) return NVFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w_bf16, 16)) return NVFP4_ERR_ALIGN;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::Bf16Args a;
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.w = static_cast<const uint16_t*>(w_bf16);
  a.M = M;
  a.N = N;
  a.K = K;
  a.num_groups = num_groups;
  a.group_offsets = num_groups > 1 ? group_offsets : nullptr;
  a.y_f32 = y_f32;
  a.y_bf16 = y_bf16;
  a.ld_y = ld_y;
  return launched(nvfp4::launch_bf16(a, stream));
}

}  // extern "C"
