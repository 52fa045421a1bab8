// k_wquant.hip — per-tensor absmean ternarisation of a weight matrix and 2-bit packing.
//
// BitNet v2 write-up, section H-BitLinear模塊: the weights are ternarised to {-1, 0, 1}
// with a per-tensor absmean scale; bitnet.cpp article, section "6 页论文，引入 1 bit LLM":
// divide the matrix by its mean absolute value and round to the nearest integer in
// {-1, 0, 1}.  The mean is summed in a fixed order (fp64, each row ascending in k, then
// the row sums ascending in n) so the scale is reproducible bit for bit.
//
// This runs once per weight matrix, outside the per-token path; it is three launches:
//   wq_rowsum   one thread per weight row, sequential fp64 sum of |W| over k
//   wq_scale    one thread: ordered sum of the row sums, alpha = max((float)(S/(N K)), 1e-5)
//   wq_pack     one thread per 16-weight word: t = clamp(rint(W/alpha), -1, 1), 2-bit fields
#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

__global__ __launch_bounds__(256) void wq_rowsum(const float* __restrict__ W, int64_t N, int64_t K,
                                                 double* __restrict__ rowsum) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const float4* p = reinterpret_cast<const float4*>(W + n * K);
  double s = 0.0;
  const int64_t k4 = K / 4;
  for (int64_t i = 0; i < k4; ++i) {
    float4 f = p[i];
    s += (double)fabsf(f.x);
    s += (double)fabsf(f.y);
    s += (double)fabsf(f.z);
    s += (double)fabsf(f.w);
  }
  rowsum[n] = s;
}

__global__ void wq_scale(const double* __restrict__ rowsum, int64_t N, int64_t K, float* __restrict__ w_scale) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double S = 0.0;
  for (int64_t n = 0; n < N; ++n) S += rowsum[n];
  float alpha = (float)(S / ((double)N * (double)K));
  if (!(alpha >= 1e-5f)) alpha = 1e-5f;
  w_scale[0] = alpha;
}

// Field position of weight c (0..15) inside its 32-bit word: p = 4*(c%4) + c/4.  With this
// order, shifting the word left by 6, 4, 2, 0 and masking 0xC0C0C0C0 yields four int8
// registers whose byte b holds 64*t for weights c = 4j + b, j = 0..3, in natural order.
__global__ __launch_bounds__(256) void wq_pack(const float* __restrict__ W, int64_t words,
                                               const float* __restrict__ w_scale, uint32_t* __restrict__ Wq) {
  const float alpha = w_scale[0];
  for (int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x; w < words; w += (int64_t)gridDim.x * 256) {
    const float4* p = reinterpret_cast<const float4*>(W + 16 * w);
    float e[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 f = p[i];
      e[4 * i + 0] = f.x;
      e[4 * i + 1] = f.y;
      e[4 * i + 2] = f.z;
      e[4 * i + 3] = f.w;
    }
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      float r = __builtin_rintf(e[c] / alpha);
      r = fminf(fmaxf(r, -1.0f), 1.0f);
      uint32_t field = (uint32_t)(int)r & 3u;
      word |= field << (2 * (4 * (c & 3) + (c >> 2)));
    }
    Wq[w] = word;
  }
}

}  // namespace

hipError_t launch_wquant(const float* W, int64_t N, int64_t K, uint8_t* Wq, float* w_scale, double* ws,
                         hipStream_t s) {
  hipLaunchKernelGGL(wq_rowsum, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, W, N, K, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wq_scale, dim3(1), dim3(64), 0, s, ws, N, K, w_scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t words = N * K / 16;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(wq_pack, dim3((unsigned)blocks), dim3(256), 0, s, W, words, w_scale,
                     reinterpret_cast<uint32_t*>(Wq));
  return hipGetLastError();
}

}  // namespace hbl
