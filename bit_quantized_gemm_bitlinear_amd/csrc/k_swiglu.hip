// k_swiglu.hip — the SwiGLU gate of the BitNet v2 FFN block, h = silu(g) * u.
//
// BitNet v2 write-up, section "BitNet v2：原生4位激活": the model is built from LLaMA-like
// parts (RMS normalisation, SwishGLU, no biases); the FFN's down projection Wdown is the
// H-BitLinear that consumes h.  silu(v) = v / (1 + exp(-v)), evaluated in fp32 with the
// exponential and reciprocal instructions (silu_mul; a few ulp from the correctly rounded
// value).
#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ g, const float* __restrict__ u,
                                                int64_t n, float* __restrict__ h) {
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 a = reinterpret_cast<const float4*>(g)[i];
    const float4 b = reinterpret_cast<const float4*>(u)[i];
    reinterpret_cast<float4*>(h)[i] =
        make_float4(silu_mul(a.x, b.x), silu_mul(a.y, b.y), silu_mul(a.z, b.z), silu_mul(a.w, b.w));
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) h[i] = silu_mul(g[i], u[i]);
}

}  // namespace

hipError_t launch_swiglu(const float* g, const float* u, int64_t n, float* h, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_swiglu, dim3((unsigned)blocks), dim3(256), 0, s, g, u, n, h);
  return hipGetLastError();
}

}  // namespace hbl
