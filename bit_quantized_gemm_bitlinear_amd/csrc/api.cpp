// api.cpp — the C ABI of libhbl (declared in include/hbl.h): synchronous argument
// validation, workspace carving and dispatch to the HIP kernels.  No HIP call happens
// before every argument has been checked, so validation is testable on a host without a
// GPU.  No exception crosses the ABI.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "hbl.h"
#include "hbl_internal.h"

namespace {

thread_local std::string g_last_error;

hbl_status fail(hbl_status s, const char* fn, const std::string& what) {
  g_last_error = std::string(fn) + ": " + what;
  return s;
}

hbl_status hip_fail(const char* fn, hipError_t e) {
  g_last_error = std::string(fn) + ": HIP error " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
  return HBL_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Shared checks of (M, K, N, abits).  N < 0 means "no N in this call".
hbl_status check_shape(const char* fn, int64_t M, int64_t K, int64_t N, int abits) {
  if (M < 0 || M > INT32_MAX) return fail(HBL_ERR_INVALID_ARG, fn, "M must be in [0, 2^31)");
  if (N != -1 && (N < 1 || N > INT32_MAX)) return fail(HBL_ERR_INVALID_ARG, fn, "N must be in [1, 2^31)");
  if (K < 64 || K % 64 != 0) return fail(HBL_ERR_INVALID_ARG, fn, "K must be a positive multiple of 64");
  if (K > HBL_MAX_K) return fail(HBL_ERR_UNSUPPORTED, fn, "K above HBL_MAX_K");
  if (abits != 4 && abits != 8) return fail(HBL_ERR_INVALID_ARG, fn, "abits must be 4 or 8");
  if (M * K > INT64_MAX / 8) return fail(HBL_ERR_INVALID_ARG, fn, "M*K too large");
  return HBL_OK;
}

hbl_status check_ptr(const char* fn, const void* p, const char* name, uintptr_t align) {
  if (p == nullptr) return fail(HBL_ERR_INVALID_ARG, fn, std::string(name) + " is NULL");
  if (!aligned(p, align))
    return fail(HBL_ERR_INVALID_ARG, fn, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return HBL_OK;
}

hbl_status check_act(const char* fn, hbl_dtype xt, hbl_norm norm, const float* gamma, float eps, int use_h,
                     int64_t K) {
  if (xt != HBL_F32 && xt != HBL_BF16) return fail(HBL_ERR_INVALID_ARG, fn, "unknown activation dtype");
  if (norm != HBL_NORM_NONE && norm != HBL_NORM_RMS) return fail(HBL_ERR_INVALID_ARG, fn, "unknown norm");
  if (norm == HBL_NORM_RMS && !(std::isfinite(eps) && eps >= 0.0f))
    return fail(HBL_ERR_INVALID_ARG, fn, "norm_eps must be finite and >= 0");
  if (norm == HBL_NORM_RMS && gamma != nullptr && !aligned(gamma, 16))
    return fail(HBL_ERR_INVALID_ARG, fn, "gamma is not 16-byte aligned");
  if (use_h != 0 && use_h != 1) return fail(HBL_ERR_INVALID_ARG, fn, "use_hadamard must be 0 or 1");
  if (use_h && !pow2(K)) return fail(HBL_ERR_UNSUPPORTED, fn, "the Hadamard transform needs K a power of two");
  if (use_h && K > HBL_MAX_K_HADAMARD) return fail(HBL_ERR_UNSUPPORTED, fn, "K above HBL_MAX_K_HADAMARD");
  return HBL_OK;
}

#define HBL_TRY(expr)              \
  do {                             \
    hbl_status st_ = (expr);       \
    if (st_ != HBL_OK) return st_; \
  } while (0)

// The forward's launches once its arguments are validated: codes and deq of the M rows go
// to ws (hbl_forward_workspace_bytes(M, K, abits) bytes, 256-byte aligned).
hbl_status run_forward(const char* fn, const void* x, hbl_dtype xt, const uint8_t* Wq, const float* w_scale,
                       int64_t M, int64_t K, int64_t N, int abits, int use_hadamard, hbl_norm norm,
                       const float* gamma, float norm_eps, float* y, void* ws, void* stream) {
  uint8_t* codes = static_cast<uint8_t*>(ws);
  float* deq = reinterpret_cast<float*>(codes + round256((size_t)(M * K * abits / 8)));
  hipStream_t s = (hipStream_t)stream;
  const float* g = norm == HBL_NORM_RMS ? gamma : nullptr;
  if (hbl::decode_fused_ok(M, K, abits, use_hadamard)) {  // a few rows: one fused kernel
    hipError_t e = hbl::launch_decode_fused(x, (int)xt, M, K, (int)norm, g, norm_eps, abits, Wq, w_scale, N, codes,
                                            deq, y, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  }
  hipError_t e = hbl::launch_actquant(x, (int)xt, M, K, (int)norm, g, norm_eps, abits, use_hadamard, codes, deq, s);
  if (e != hipSuccess) return hip_fail(fn, e);
  e = hbl::launch_gemm(codes, deq, Wq, w_scale, M, K, N, abits, nullptr, y, s);
  if (e != hipSuccess) return hip_fail(fn, e);
  return HBL_OK;
}

}  // namespace

// Scratch of hbl_forward_noalloc: the codes and deq of one call, in a device array that the
// library owns (one copy per GPU, alive until the process ends).  Host code never passes the
// array's name to a kernel: the name is a host-side stand-in, not a device address.  It uses
// the address hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[HBL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int hbl_version(void) { return 100; }

const char* hbl_status_string(hbl_status s) {
  switch (s) {
    case HBL_OK: return "HBL_OK";
    case HBL_ERR_INVALID_ARG: return "HBL_ERR_INVALID_ARG";
    case HBL_ERR_UNSUPPORTED: return "HBL_ERR_UNSUPPORTED";
    case HBL_ERR_WORKSPACE: return "HBL_ERR_WORKSPACE";
    case HBL_ERR_HIP: return "HBL_ERR_HIP";
  }
  return "HBL_ERR_UNKNOWN";
}

const char* hbl_last_error(void) { return g_last_error.c_str(); }

size_t hbl_packed_weight_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 64 || K % 64 != 0 || K > HBL_MAX_K || N > INT32_MAX) return 0;
  return (size_t)(N * (K / 4));
}

size_t hbl_packed_act_bytes(int64_t M, int64_t K, int abits) {
  if (M < 0 || K < 64 || K % 64 != 0 || K > HBL_MAX_K || M > INT32_MAX || (abits != 4 && abits != 8)) return 0;
  return (size_t)(M * K * abits / 8);
}

size_t hbl_wquant_workspace_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 64 || K % 64 != 0 || K > HBL_MAX_K || N > INT32_MAX) return 0;
  return (size_t)N * sizeof(double);
}

size_t hbl_forward_workspace_bytes(int64_t M, int64_t K, int abits) {
  if (M < 0 || K < 64 || K % 64 != 0 || K > HBL_MAX_K || M > INT32_MAX || (abits != 4 && abits != 8)) return 0;
  return round256((size_t)(M * K * abits / 8)) + round256((size_t)M * sizeof(float));
}

hbl_status hbl_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* Wq, float* w_scale, void* ws,
                                size_t ws_bytes, void* stream) {
  static const char* fn = "hbl_quantize_weights";
  try {
    if (N < 1 || N > INT32_MAX) return fail(HBL_ERR_INVALID_ARG, fn, "N must be in [1, 2^31)");
    HBL_TRY(check_shape(fn, 0, K, N, 4));
    HBL_TRY(check_ptr(fn, W, "W", 16));
    HBL_TRY(check_ptr(fn, Wq, "Wq", 16));
    HBL_TRY(check_ptr(fn, w_scale, "w_scale", 4));
    if (ws == nullptr || ws_bytes < hbl_wquant_workspace_bytes(N, K))
      return fail(HBL_ERR_WORKSPACE, fn, "workspace missing or smaller than hbl_wquant_workspace_bytes");
    HBL_TRY(check_ptr(fn, ws, "ws", 16));
    hipError_t e = hbl::launch_wquant(W, N, K, Wq, w_scale, static_cast<double*>(ws), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_quantize_activations(const void* x, hbl_dtype xt, int64_t M, int64_t K, hbl_norm norm,
                                    const float* gamma, float norm_eps, int abits, int use_hadamard, uint8_t* codes,
                                    float* deq, void* stream) {
  static const char* fn = "hbl_quantize_activations";
  try {
    HBL_TRY(check_shape(fn, M, K, -1, abits));
    HBL_TRY(check_act(fn, xt, norm, gamma, norm_eps, use_hadamard, K));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, codes, "codes", 16));
    HBL_TRY(check_ptr(fn, deq, "deq", 4));
    hipError_t e = hbl::launch_actquant(x, (int)xt, M, K, (int)norm, norm == HBL_NORM_RMS ? gamma : nullptr,
                                        norm_eps, abits, use_hadamard, codes, deq, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_gemm_s32(const uint8_t* codes, const uint8_t* Wq, int64_t M, int64_t K, int64_t N, int abits,
                        int32_t* acc, void* stream) {
  static const char* fn = "hbl_gemm_s32";
  try {
    HBL_TRY(check_shape(fn, M, K, N, abits));
    HBL_TRY(check_ptr(fn, Wq, "Wq", 16));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, codes, "codes", 16));
    HBL_TRY(check_ptr(fn, acc, "acc", 16));
    hipError_t e = hbl::launch_gemm(codes, nullptr, Wq, nullptr, M, K, N, abits, acc, nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_gemm_dequant(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale,
                            int64_t M, int64_t K, int64_t N, int abits, float* y, void* stream) {
  static const char* fn = "hbl_gemm_dequant";
  try {
    HBL_TRY(check_shape(fn, M, K, N, abits));
    HBL_TRY(check_ptr(fn, Wq, "Wq", 16));
    HBL_TRY(check_ptr(fn, w_scale, "w_scale", 4));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, codes, "codes", 16));
    HBL_TRY(check_ptr(fn, deq, "deq", 4));
    HBL_TRY(check_ptr(fn, y, "y", 16));
    hipError_t e = hbl::launch_gemm(codes, deq, Wq, w_scale, M, K, N, abits, nullptr, y, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_forward(const void* x, hbl_dtype xt, const uint8_t* Wq, const float* w_scale, int64_t M, int64_t K,
                       int64_t N, int abits, int use_hadamard, hbl_norm norm, const float* gamma, float norm_eps,
                       float* y, void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "hbl_forward";
  try {
    HBL_TRY(check_shape(fn, M, K, N, abits));
    HBL_TRY(check_act(fn, xt, norm, gamma, norm_eps, use_hadamard, K));
    HBL_TRY(check_ptr(fn, Wq, "Wq", 16));
    HBL_TRY(check_ptr(fn, w_scale, "w_scale", 4));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, y, "y", 16));
    const size_t need = hbl_forward_workspace_bytes(M, K, abits);
    if (ws == nullptr || ws_bytes < need)
      return fail(HBL_ERR_WORKSPACE, fn, "workspace missing or smaller than hbl_forward_workspace_bytes");
    HBL_TRY(check_ptr(fn, ws, "ws", 256));
    return run_forward(fn, x, xt, Wq, w_scale, M, K, N, abits, use_hadamard, norm, gamma, norm_eps, y, ws, stream);
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_forward_noalloc(const void* x, hbl_dtype xt, const uint8_t* Wq, const float* w_scale, int64_t M,
                               int64_t K, int64_t N, int abits, int use_hadamard, hbl_norm norm, const float* gamma,
                               float norm_eps, float* y, void* stream) {
  static const char* fn = "hbl_forward_noalloc";
  try {
    HBL_TRY(check_shape(fn, M, K, N, abits));
    HBL_TRY(check_act(fn, xt, norm, gamma, norm_eps, use_hadamard, K));
    HBL_TRY(check_ptr(fn, Wq, "Wq", 16));
    HBL_TRY(check_ptr(fn, w_scale, "w_scale", 4));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, y, "y", 16));
    const size_t need = hbl_forward_workspace_bytes(M, K, abits);
    if (need > (size_t)HBL_NOALLOC_SCRATCH_BYTES)
      return fail(HBL_ERR_UNSUPPORTED, fn,
                  "the codes and deq of this call need " + std::to_string(need) +
                      " bytes, above the static scratch of HBL_NOALLOC_SCRATCH_BYTES = " +
                      std::to_string((size_t)HBL_NOALLOC_SCRATCH_BYTES) + "; use hbl_forward with a workspace");
    void* ws = nullptr;
    hipError_t e = scratch_of_current_device(&ws);
    if (e != hipSuccess) return hip_fail(fn, e);
    return run_forward(fn, x, xt, Wq, w_scale, M, K, N, abits, use_hadamard, norm, gamma, norm_eps, y, ws, stream);
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_quantize_activations_stat(const void* x, hbl_dtype xt, int64_t M, int64_t K, hbl_norm norm,
                                         const float* gamma, float norm_eps, int abits, int use_hadamard, int stat,
                                         uint8_t* codes, float* deq, void* stream) {
  static const char* fn = "hbl_quantize_activations_stat";
  try {
    if (stat != HBL_STAT_ABSMAX && stat != HBL_STAT_ABSMEAN) return fail(HBL_ERR_INVALID_ARG, fn, "unknown stat");
    if (stat == HBL_STAT_ABSMEAN && abits != 4)
      return fail(HBL_ERR_UNSUPPORTED, fn, "the absmean statistic is implemented for abits = 4");
    HBL_TRY(check_shape(fn, M, K, -1, abits));
    HBL_TRY(check_act(fn, xt, norm, gamma, norm_eps, use_hadamard, K));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, codes, "codes", 16));
    HBL_TRY(check_ptr(fn, deq, "deq", 4));
    hipError_t e = hbl::launch_actquant(x, (int)xt, M, K, (int)norm, norm == HBL_NORM_RMS ? gamma : nullptr,
                                        norm_eps, stat == HBL_STAT_ABSMEAN ? 5 : abits, use_hadamard, codes, deq,
                                        (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_forward_stat(const void* x, hbl_dtype xt, const uint8_t* Wq, const float* w_scale, int64_t M,
                            int64_t K, int64_t N, int abits, int use_hadamard, hbl_norm norm, const float* gamma,
                            float norm_eps, int stat, float* y, void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "hbl_forward_stat";
  try {
    if (stat == HBL_STAT_ABSMAX)
      return hbl_forward(x, xt, Wq, w_scale, M, K, N, abits, use_hadamard, norm, gamma, norm_eps, y, ws, ws_bytes,
                         stream);
    if (stat != HBL_STAT_ABSMEAN) return fail(HBL_ERR_INVALID_ARG, fn, "unknown stat");
    if (abits != 4) return fail(HBL_ERR_UNSUPPORTED, fn, "the absmean statistic is implemented for abits = 4");
    HBL_TRY(check_shape(fn, M, K, N, abits));
    HBL_TRY(check_act(fn, xt, norm, gamma, norm_eps, use_hadamard, K));
    HBL_TRY(check_ptr(fn, Wq, "Wq", 16));
    HBL_TRY(check_ptr(fn, w_scale, "w_scale", 4));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, y, "y", 16));
    if (ws == nullptr || ws_bytes < hbl_forward_workspace_bytes(M, K, abits))
      return fail(HBL_ERR_WORKSPACE, fn, "workspace missing or smaller than hbl_forward_workspace_bytes");
    HBL_TRY(check_ptr(fn, ws, "ws", 256));
    uint8_t* codes = static_cast<uint8_t*>(ws);
    float* deq = reinterpret_cast<float*>(codes + round256((size_t)(M * K * abits / 8)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hbl::launch_actquant(x, (int)xt, M, K, (int)norm, norm == HBL_NORM_RMS ? gamma : nullptr,
                                        norm_eps, 5, use_hadamard, codes, deq, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    e = hbl::launch_gemm(codes, deq, Wq, w_scale, M, K, N, 4, nullptr, y, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

size_t hbl_packed_weight_fp4_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 64 || K % 64 != 0 || K > HBL_MAX_K || N > INT32_MAX) return 0;
  return (size_t)(N * (K / 2));
}

size_t hbl_packed_act_fp6_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 64 || K % 64 != 0 || K > HBL_MAX_K || M > INT32_MAX) return 0;
  return (size_t)(M * (K / 4) * 3);
}

size_t hbl_forward_fp6fp4_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 64 || K % 64 != 0 || K > HBL_MAX_K || M > INT32_MAX) return 0;
  return round256((size_t)(M * (K / 4) * 3)) + round256((size_t)M * sizeof(float));
}

hbl_status hbl_weights_to_fp4(const uint8_t* Wq, int64_t N, int64_t K, uint8_t* Wq4, void* stream) {
  static const char* fn = "hbl_weights_to_fp4";
  try {
    if (N < 1 || N > INT32_MAX) return fail(HBL_ERR_INVALID_ARG, fn, "N must be in [1, 2^31)");
    HBL_TRY(check_shape(fn, 0, K, N, 4));
    HBL_TRY(check_ptr(fn, Wq, "Wq", 16));
    HBL_TRY(check_ptr(fn, Wq4, "Wq4", 16));
    hipError_t e = hbl::launch_weights_fp4(Wq, N, K, Wq4, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_quantize_activations_fp6(const void* x, hbl_dtype xt, int64_t M, int64_t K, hbl_norm norm,
                                        const float* gamma, float norm_eps, int use_hadamard, uint8_t* codes6,
                                        float* deq, void* stream) {
  static const char* fn = "hbl_quantize_activations_fp6";
  try {
    HBL_TRY(check_shape(fn, M, K, -1, 4));
    HBL_TRY(check_act(fn, xt, norm, gamma, norm_eps, use_hadamard, K));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, codes6, "codes6", 16));
    HBL_TRY(check_ptr(fn, deq, "deq", 4));
    hipError_t e = hbl::launch_actquant(x, (int)xt, M, K, (int)norm, norm == HBL_NORM_RMS ? gamma : nullptr,
                                        norm_eps, 6, use_hadamard, codes6, deq, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_gemm_fp6fp4_s32(const uint8_t* codes6, const uint8_t* Wq4, int64_t M, int64_t K, int64_t N,
                               int32_t* acc, void* stream) {
  static const char* fn = "hbl_gemm_fp6fp4_s32";
  try {
    HBL_TRY(check_shape(fn, M, K, N, 4));
    HBL_TRY(check_ptr(fn, Wq4, "Wq4", 16));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, codes6, "codes6", 16));
    HBL_TRY(check_ptr(fn, acc, "acc", 16));
    hipError_t e = hbl::launch_gemm_f6f4(codes6, nullptr, Wq4, nullptr, M, K, N, acc, nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_gemm_fp6fp4_dequant(const uint8_t* codes6, const float* deq, const uint8_t* Wq4, const float* w_scale,
                                   int64_t M, int64_t K, int64_t N, float* y, void* stream) {
  static const char* fn = "hbl_gemm_fp6fp4_dequant";
  try {
    HBL_TRY(check_shape(fn, M, K, N, 4));
    HBL_TRY(check_ptr(fn, Wq4, "Wq4", 16));
    HBL_TRY(check_ptr(fn, w_scale, "w_scale", 4));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, codes6, "codes6", 16));
    HBL_TRY(check_ptr(fn, deq, "deq", 4));
    HBL_TRY(check_ptr(fn, y, "y", 16));
    hipError_t e = hbl::launch_gemm_f6f4(codes6, deq, Wq4, w_scale, M, K, N, nullptr, y, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_forward_fp6fp4(const void* x, hbl_dtype xt, const uint8_t* Wq4, const float* w_scale, int64_t M,
                              int64_t K, int64_t N, int use_hadamard, hbl_norm norm, const float* gamma,
                              float norm_eps, float* y, void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "hbl_forward_fp6fp4";
  try {
    HBL_TRY(check_shape(fn, M, K, N, 4));
    HBL_TRY(check_act(fn, xt, norm, gamma, norm_eps, use_hadamard, K));
    HBL_TRY(check_ptr(fn, Wq4, "Wq4", 16));
    HBL_TRY(check_ptr(fn, w_scale, "w_scale", 4));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, y, "y", 16));
    const size_t need = hbl_forward_fp6fp4_workspace_bytes(M, K);
    if (ws == nullptr || ws_bytes < need)
      return fail(HBL_ERR_WORKSPACE, fn, "workspace missing or smaller than hbl_forward_fp6fp4_workspace_bytes");
    HBL_TRY(check_ptr(fn, ws, "ws", 256));
    uint8_t* codes = static_cast<uint8_t*>(ws);
    float* deq = reinterpret_cast<float*>(codes + round256((size_t)(M * (K / 4) * 3)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hbl::launch_actquant(x, (int)xt, M, K, (int)norm, norm == HBL_NORM_RMS ? gamma : nullptr,
                                        norm_eps, 6, use_hadamard, codes, deq, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    e = hbl::launch_gemm_f6f4(codes, deq, Wq4, w_scale, M, K, N, nullptr, y, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

size_t hbl_packed_gate_up_bytes(int64_t F, int64_t K) {
  if (F < 32 || F % 32 != 0 || 2 * F > INT32_MAX || K < 64 || K % 64 != 0 || K > HBL_MAX_K) return 0;
  return (size_t)(2 * F * (K / 4));
}

hbl_status hbl_interleave_gate_up(const uint8_t* Wq_gate, const uint8_t* Wq_up, int64_t F, int64_t K, uint8_t* Wgu,
                                  void* stream) {
  static const char* fn = "hbl_interleave_gate_up";
  try {
    if (F < 32 || F % 32 != 0 || 2 * F > INT32_MAX)
      return fail(HBL_ERR_INVALID_ARG, fn, "F must be a positive multiple of 32 below 2^30");
    HBL_TRY(check_shape(fn, 0, K, 2 * F, 4));
    HBL_TRY(check_ptr(fn, Wq_gate, "Wq_gate", 16));
    HBL_TRY(check_ptr(fn, Wq_up, "Wq_up", 16));
    HBL_TRY(check_ptr(fn, Wgu, "Wgu", 16));
    const size_t row = (size_t)(K / 4), blk = 32 * row;
    const uintptr_t ob = reinterpret_cast<uintptr_t>(Wgu), oe = ob + 2 * (size_t)F * row;
    for (const uint8_t* p : {Wq_gate, Wq_up}) {
      const uintptr_t pb = reinterpret_cast<uintptr_t>(p), pe = pb + (size_t)F * row;
      if (ob < pe && pb < oe) return fail(HBL_ERR_INVALID_ARG, fn, "Wgu overlaps an input");
    }
    hipStream_t s = (hipStream_t)stream;
    // Block b of 32 gate rows goes to rows 64b..64b+31, the matching up rows to 64b+32..64b+63.
    hipError_t e = hipMemcpy2DAsync(Wgu, 2 * blk, Wq_gate, blk, blk, (size_t)(F / 32), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    e = hipMemcpy2DAsync(Wgu + blk, 2 * blk, Wq_up, blk, blk, (size_t)(F / 32), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_gate_up_swiglu(const uint8_t* codes, const float* deq, const uint8_t* Wgu, const float* scale_gate,
                              const float* scale_up, int64_t M, int64_t K, int64_t F, int abits, hbl_dtype ht, void* h,
                              void* stream) {
  static const char* fn = "hbl_gate_up_swiglu";
  try {
    if (F < 32 || F % 32 != 0 || 2 * F > INT32_MAX)
      return fail(HBL_ERR_INVALID_ARG, fn, "F must be a positive multiple of 32 below 2^30");
    HBL_TRY(check_shape(fn, M, K, 2 * F, abits));
    if (ht != HBL_F32 && ht != HBL_BF16) return fail(HBL_ERR_INVALID_ARG, fn, "unknown h dtype");
    HBL_TRY(check_ptr(fn, Wgu, "Wgu", 16));
    HBL_TRY(check_ptr(fn, scale_gate, "scale_gate", 4));
    HBL_TRY(check_ptr(fn, scale_up, "scale_up", 4));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, codes, "codes", 16));
    HBL_TRY(check_ptr(fn, deq, "deq", 4));
    HBL_TRY(check_ptr(fn, h, "h", 16));
    hipError_t e = hbl::launch_gemm_swiglu(codes, deq, Wgu, scale_gate, scale_up, M, K, F, abits, ht == HBL_BF16, h,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

size_t hbl_ffn_workspace_bytes(int64_t M, int64_t D, int64_t F, int abits, hbl_dtype ht) {
  if (M < 0 || M > INT32_MAX || D < 64 || D % 64 != 0 || D > HBL_MAX_K || !pow2(F) || F < 64 ||
      F > HBL_MAX_K_HADAMARD || (abits != 4 && abits != 8) || (ht != HBL_F32 && ht != HBL_BF16))
    return 0;
  const size_t hb = ht == HBL_BF16 ? 2 : 4;
  return round256((size_t)(M * D * abits / 8)) + round256((size_t)M * sizeof(float)) + round256((size_t)(M * F) * hb) +
         hbl_forward_workspace_bytes(M, F, abits);
}

hbl_status hbl_ffn_forward(const void* x, hbl_dtype xt, const uint8_t* Wgu, const float* scale_gate,
                           const float* scale_up, const uint8_t* Wq_down, const float* scale_down, int64_t M, int64_t D,
                           int64_t F, int abits, const float* gamma_in, const float* gamma_down, float norm_eps,
                           hbl_dtype ht, float* y, void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "hbl_ffn_forward";
  try {
    HBL_TRY(check_shape(fn, M, D, 2 * F, abits));
    HBL_TRY(check_shape(fn, M, F, D, abits));
    HBL_TRY(check_act(fn, xt, HBL_NORM_RMS, gamma_in, norm_eps, 0, D));
    if (ht != HBL_F32 && ht != HBL_BF16) return fail(HBL_ERR_INVALID_ARG, fn, "unknown h dtype");
    HBL_TRY(check_act(fn, ht, HBL_NORM_RMS, gamma_down, norm_eps, 1, F));
    HBL_TRY(check_ptr(fn, Wgu, "Wgu", 16));
    HBL_TRY(check_ptr(fn, scale_gate, "scale_gate", 4));
    HBL_TRY(check_ptr(fn, scale_up, "scale_up", 4));
    HBL_TRY(check_ptr(fn, Wq_down, "Wq_down", 16));
    HBL_TRY(check_ptr(fn, scale_down, "scale_down", 4));
    if (M == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, y, "y", 16));
    const size_t need = hbl_ffn_workspace_bytes(M, D, F, abits, ht);
    if (ws == nullptr || ws_bytes < need)
      return fail(HBL_ERR_WORKSPACE, fn, "workspace missing or smaller than hbl_ffn_workspace_bytes");
    HBL_TRY(check_ptr(fn, ws, "ws", 256));
    uint8_t* codes = static_cast<uint8_t*>(ws);
    float* deq = reinterpret_cast<float*>(codes + round256((size_t)(M * D * abits / 8)));
    uint8_t* h = reinterpret_cast<uint8_t*>(deq) + round256((size_t)M * sizeof(float));
    uint8_t* codes2 = h + round256((size_t)(M * F) * (ht == HBL_BF16 ? 2 : 4));
    float* deq2 = reinterpret_cast<float*>(codes2 + round256((size_t)(M * F * abits / 8)));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hbl::launch_actquant(x, (int)xt, M, D, (int)HBL_NORM_RMS, gamma_in, norm_eps, abits, 0, codes, deq, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    e = hbl::launch_gemm_swiglu(codes, deq, Wgu, scale_gate, scale_up, M, D, F, abits, ht == HBL_BF16, h, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    e = hbl::launch_actquant(h, (int)ht, M, F, (int)HBL_NORM_RMS, gamma_down, norm_eps, abits, 1, codes2, deq2, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    e = hbl::launch_gemm(codes2, deq2, Wq_down, scale_down, M, F, D, abits, nullptr, y, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

namespace {
hbl_status check_qkv(const char* fn, int64_t rows, int64_t d, int bits) {
  if (rows < 0 || rows > INT32_MAX) return fail(HBL_ERR_INVALID_ARG, fn, "rows must be in [0, 2^31)");
  if (bits < 2 || bits > 8) return fail(HBL_ERR_INVALID_ARG, fn, "bits must be in 2..8");
  if (d != 32 && d != 64 && d != 128 && d != 256 && d != 512)
    return fail(HBL_ERR_UNSUPPORTED, fn, "head size d must be 32, 64, 128, 256 or 512");
  return HBL_OK;
}
}  // namespace

size_t hbl_packed_qkv_bytes(int64_t rows, int64_t d, int bits) {
  if (rows < 0 || rows > INT32_MAX || bits < 2 || bits > 8 ||
      (d != 32 && d != 64 && d != 128 && d != 256 && d != 512))
    return 0;
  return (size_t)(rows * d * bits / 8);
}

hbl_status hbl_quantize_qkv(const void* x, hbl_dtype xt, int64_t rows, int64_t d, int bits, uint8_t* codes,
                            float* gamma, void* stream) {
  static const char* fn = "hbl_quantize_qkv";
  try {
    HBL_TRY(check_qkv(fn, rows, d, bits));
    if (xt != HBL_F32 && xt != HBL_BF16) return fail(HBL_ERR_INVALID_ARG, fn, "unknown dtype");
    if (rows == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, x, "x", 16));
    HBL_TRY(check_ptr(fn, codes, "codes", 16));
    HBL_TRY(check_ptr(fn, gamma, "gamma", 4));
    hipError_t e = hbl::launch_qkv_quant(x, (int)xt, rows, d, bits, codes, gamma, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

hbl_status hbl_dequantize_qkv(const uint8_t* codes, const float* gamma, int64_t rows, int64_t d, int bits, float* out,
                              void* stream) {
  static const char* fn = "hbl_dequantize_qkv";
  try {
    HBL_TRY(check_qkv(fn, rows, d, bits));
    if (rows == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, codes, "codes", 16));
    HBL_TRY(check_ptr(fn, gamma, "gamma", 4));
    HBL_TRY(check_ptr(fn, out, "out", 16));
    hipError_t e = hbl::launch_qkv_dequant(codes, gamma, rows, d, bits, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

int hbl_forward_fused(int64_t M, int64_t K, int abits, int use_hadamard) {
  if (M < 1 || K < 64 || K % 64 != 0 || K > HBL_MAX_K || (use_hadamard != 0 && use_hadamard != 1)) return 0;
  if (use_hadamard && !pow2(K)) return 0;
  return hbl::decode_fused_ok(M, K, abits, use_hadamard) ? 1 : 0;
}

hbl_status hbl_swiglu(const float* g, const float* u, int64_t n, float* h, void* stream) {
  static const char* fn = "hbl_swiglu";
  try {
    if (n < 0) return fail(HBL_ERR_INVALID_ARG, fn, "n must be >= 0");
    if (n == 0) return HBL_OK;
    HBL_TRY(check_ptr(fn, g, "g", 16));
    HBL_TRY(check_ptr(fn, u, "u", 16));
    HBL_TRY(check_ptr(fn, h, "h", 16));
    const uintptr_t hb = reinterpret_cast<uintptr_t>(h), he = hb + (uintptr_t)n * sizeof(float);
    for (const float* p : {g, u}) {
      const uintptr_t pb = reinterpret_cast<uintptr_t>(p), pe = pb + (uintptr_t)n * sizeof(float);
      if (hb < pe && pb < he) return fail(HBL_ERR_INVALID_ARG, fn, "h overlaps an input");
    }
    hipError_t e = hbl::launch_swiglu(g, u, n, h, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return HBL_OK;
  } catch (...) {
    return fail(HBL_ERR_HIP, fn, "unexpected C++ exception");
  }
}

}  // extern "C"
