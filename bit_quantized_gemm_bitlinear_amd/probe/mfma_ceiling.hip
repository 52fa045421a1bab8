// mfma_ceiling.hip — a measurement aid, not part of the layer.  It measures the int8
// matrix-core rate this GPU sustains with nothing else to do: no memory traffic, no VALU,
// no LDS.  The GEMM's achieved rate is reported against it beside the published peak,
// which assumes the peak clock; under MFMA load the clock sags.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Each wave runs `iters` rounds of four independent v_mfma_i32_32x32x32_i8 chains on operands
// loaded from `ops` (2 x 64 lanes x 16 bytes; the operand bits matter, since the matrix
// cores' power depends on them), then stores a checksum so the work is kept.
__global__ __launch_bounds__(256) void k_mfma_ceiling(const v4i* __restrict__ ops, int iters, int* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const v4i a = ops[lane], b = ops[64 + lane];
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// The same for v_mfma_scale_f32_32x32x64_f8f6f4 with A in FP6 E2M3 (6 registers used) and B
// in FP4 E2M1 (4 registers used), block scales 2^0, as the FP6 x FP4 GEMM issues it.
__global__ __launch_bounds__(256) void k_mfma_f6f4_ceiling(const v8i* __restrict__ ops, int iters,
                                                           int* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  v8i a = ops[lane], b = ops[64 + lane];
  a[6] = a[7] = 0;
  b[4] = b[5] = b[6] = b[7] = 0;
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 2, 4, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 2, 4, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 2, 4, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 2, 4, 0, 127, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  out[blockIdx.x * 256 + threadIdx.x] = (int)s;
}

// The shader clock under matrix-core load: the int8 MFMA chains of k_mfma_ceiling, with the
// shader-clock counter (s_memtime) and the constant-rate counter (s_memrealtime) read by the
// first lane of each block at its start and end.  Their ratio times the constant counter's rate
// is the average clock the block ran at.
__global__ __launch_bounds__(256) void k_clock(const v4i* __restrict__ ops, int iters, int* __restrict__ out,
                                               unsigned long long* __restrict__ ts) {
  const int lane = threadIdx.x & 63;
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  const v4i a = ops[lane], b = ops[64 + lane];
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    ts[2 * blockIdx.x] = t1 - t0;
    ts[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// HBM streaming with the activation kernel's traffic mix: every 16 bytes read produce 4 bytes
// written (bf16 in, packed INT4 out), four 16-byte loads in flight per thread, grid-stride.
__global__ __launch_bounds__(256) void k_stream(const uint4* __restrict__ x, int64_t n16, uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) out[i + u * stride] = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = x[i];
    out[i] = v.x ^ v.y ^ v.z ^ v.w;
  }
}

}  // namespace

// Reads n16 16-byte chunks of x and writes n16 words of out (both device, n16 >= 1).
extern "C" int hbl_probe_stream(const void* x, int64_t n16, unsigned* out, int blocks, void* stream) {
  if (x == nullptr || out == nullptr || n16 < 1 || blocks < 1) return 1;
  hipLaunchKernelGGL(k_stream, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(x), n16, static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// ops as hbl_probe_mfma_ceiling; out: blocks * 256 ints; ts: blocks * 2 uint64 (shader-clock
// ticks, constant-rate ticks).  Returns 0 on success.
extern "C" int hbl_probe_clock(const void* ops, int blocks, int iters, int* out, unsigned long long* ts, void* stream) {
  if (ops == nullptr || out == nullptr || ts == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(k_clock, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, static_cast<const v4i*>(ops),
                     iters, out, ts);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Rate of the constant-rate counter (s_memrealtime) in kHz, or 0 if the query fails.
extern "C" int hbl_probe_wallclock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

// ops: device, 128 x 32 bytes (FP6 codes for A, FP4 weights for B); out: device, blocks * 256
// ints.  Each launch performs blocks * 4 waves * iters * 4 MFMAs of 32*32*64*2 = 131072 ops.
extern "C" int hbl_probe_mfma_f6f4_ceiling(const void* ops, int blocks, int iters, int* out, void* stream) {
  if (ops == nullptr || out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(k_mfma_f6f4_ceiling, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const v8i*>(ops), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// ops: device, 128 x 16 bytes; out: device, blocks * 256 ints.  Each launch performs
// blocks * 4 waves * iters * 4 MFMAs of 32*32*32*2 = 65536 int8 ops.  Returns 0 on success.
extern "C" int hbl_probe_mfma_ceiling(const void* ops, int blocks, int iters, int* out, void* stream) {
  if (ops == nullptr || out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(k_mfma_ceiling, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const v4i*>(ops), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
