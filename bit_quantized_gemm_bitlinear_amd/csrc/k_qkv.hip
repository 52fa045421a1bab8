// k_qkv.hip — unsigned absmax quantisation of post-RoPE Q/K/V head vectors (the low-bit
// attention states and the 3-bit KV cache of the BitNet v2 write-up, text of Tables 2 and 3)
// and its inverse.
//
// Per head vector x of length d: g = max|x|, s = L / (2g) with L = 2^BITS - 1, and
// u = clamp(rint_ne(x*s + L/2), 0, L); codes are packed least significant bit first (code i
// at bits [BITS*i, BITS*i + BITS) of the head's bit string).  Reconstruction:
// xhat = (u - L/2) * (2g / L).  Every operation is an fp32 operation in that order.
//
// One thread handles 32 consecutive values (BITS whole 32-bit words of output); the G =
// d/32 threads of a head are adjacent lanes and reduce the maximum with lane shuffles.  The
// kernel is bound by HBM traffic (read 2 or 4 bytes per value, write BITS/8).
#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

template <int XT>
__device__ __forceinline__ void load32(const void* x, int64_t off, float (&v)[32]) {
  if constexpr (XT == 0) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = p[i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16lo(ws[j]);
        v[8 * i + 2 * j + 1] = bf16hi(ws[j]);
      }
    }
  }
}

template <int BITS, int XT, int G>
__global__ __launch_bounds__(256) void k_qkv_quant(const void* __restrict__ x, int64_t rows,
                                                   uint32_t* __restrict__ codes, float* __restrict__ gamma) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / G;
  const bool live = row < rows;
  float v[32];
  if (live) load32<XT>(x, t * 32, v);
  float m = 0.0f;
  if (live) {
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  // the G lanes of a head are adjacent and G divides 64: xor shuffles stay inside the head
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (!live) return;
  constexpr float L = (float)((1 << BITS) - 1);
  constexpr float c = L / 2.0f;
  const float s = m < 0x1p-120f ? 0.0f : __fdiv_rn(L, 2.0f * m);
  uint32_t w[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float q = fminf(fmaxf(__builtin_rintf(__fadd_rn(__fmul_rn(v[i], s), c)), 0.0f), L);
    const uint32_t u = (uint32_t)q;
    const int bit = BITS * i;
    w[bit / 32] |= u << (bit % 32);
    if (bit % 32 + BITS > 32) w[bit / 32 + 1] |= u >> (32 - bit % 32);
  }
  uint32_t* out = codes + t * BITS;
#pragma unroll
  for (int i = 0; i < BITS; ++i) out[i] = w[i];
  if (t % G == 0) gamma[row] = m;
}

template <int BITS, int G>
__global__ __launch_bounds__(256) void k_qkv_dequant(const uint32_t* __restrict__ codes,
                                                     const float* __restrict__ gamma, int64_t rows,
                                                     float* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / G;
  if (row >= rows) return;
  constexpr float L = (float)((1 << BITS) - 1);
  constexpr float c = L / 2.0f;
  const float D = __fdiv_rn(2.0f * gamma[row], L);
  uint32_t w[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = codes[t * BITS + i];
  float o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int bit = BITS * i;
    uint32_t u = w[bit / 32] >> (bit % 32);
    if (bit % 32 + BITS > 32) u |= w[bit / 32 + 1] << (32 - bit % 32);
    u &= (1u << BITS) - 1u;
    o[i] = __fmul_rn((float)u - c, D);
  }
  float4* p = reinterpret_cast<float4*>(out + t * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

template <int BITS, int XT>
hipError_t quant_g(const void* x, int64_t rows, int64_t d, uint8_t* codes, float* gamma, hipStream_t s) {
  const int64_t threads = rows * (d / 32);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  uint32_t* c = reinterpret_cast<uint32_t*>(codes);
  switch (d / 32) {
    case 1: hipLaunchKernelGGL((k_qkv_quant<BITS, XT, 1>), grid, block, 0, s, x, rows, c, gamma); break;
    case 2: hipLaunchKernelGGL((k_qkv_quant<BITS, XT, 2>), grid, block, 0, s, x, rows, c, gamma); break;
    case 4: hipLaunchKernelGGL((k_qkv_quant<BITS, XT, 4>), grid, block, 0, s, x, rows, c, gamma); break;
    case 8: hipLaunchKernelGGL((k_qkv_quant<BITS, XT, 8>), grid, block, 0, s, x, rows, c, gamma); break;
    default: hipLaunchKernelGGL((k_qkv_quant<BITS, XT, 16>), grid, block, 0, s, x, rows, c, gamma); break;
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t dequant_g(const uint8_t* codes, const float* gamma, int64_t rows, int64_t d, float* out, hipStream_t s) {
  const int64_t threads = rows * (d / 32);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const uint32_t* c = reinterpret_cast<const uint32_t*>(codes);
  switch (d / 32) {
    case 1: hipLaunchKernelGGL((k_qkv_dequant<BITS, 1>), grid, block, 0, s, c, gamma, rows, out); break;
    case 2: hipLaunchKernelGGL((k_qkv_dequant<BITS, 2>), grid, block, 0, s, c, gamma, rows, out); break;
    case 4: hipLaunchKernelGGL((k_qkv_dequant<BITS, 4>), grid, block, 0, s, c, gamma, rows, out); break;
    case 8: hipLaunchKernelGGL((k_qkv_dequant<BITS, 8>), grid, block, 0, s, c, gamma, rows, out); break;
    default: hipLaunchKernelGGL((k_qkv_dequant<BITS, 16>), grid, block, 0, s, c, gamma, rows, out); break;
  }
  return hipGetLastError();
}

template <int XT>
hipError_t quant_x(const void* x, int64_t rows, int64_t d, int bits, uint8_t* codes, float* gamma, hipStream_t s) {
  switch (bits) {
    case 2: return quant_g<2, XT>(x, rows, d, codes, gamma, s);
    case 3: return quant_g<3, XT>(x, rows, d, codes, gamma, s);
    case 4: return quant_g<4, XT>(x, rows, d, codes, gamma, s);
    case 5: return quant_g<5, XT>(x, rows, d, codes, gamma, s);
    case 6: return quant_g<6, XT>(x, rows, d, codes, gamma, s);
    case 7: return quant_g<7, XT>(x, rows, d, codes, gamma, s);
    default: return quant_g<8, XT>(x, rows, d, codes, gamma, s);
  }
}

}  // namespace

hipError_t launch_qkv_quant(const void* x, int xt, int64_t rows, int64_t d, int bits, uint8_t* codes, float* gamma,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  return xt == 0 ? quant_x<0>(x, rows, d, bits, codes, gamma, s) : quant_x<1>(x, rows, d, bits, codes, gamma, s);
}

hipError_t launch_qkv_dequant(const uint8_t* codes, const float* gamma, int64_t rows, int64_t d, int bits, float* out,
                              hipStream_t s) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return dequant_g<2>(codes, gamma, rows, d, out, s);
    case 3: return dequant_g<3>(codes, gamma, rows, d, out, s);
    case 4: return dequant_g<4>(codes, gamma, rows, d, out, s);
    case 5: return dequant_g<5>(codes, gamma, rows, d, out, s);
    case 6: return dequant_g<6>(codes, gamma, rows, d, out, s);
    case 7: return dequant_g<7>(codes, gamma, rows, d, out, s);
    default: return dequant_g<8>(codes, gamma, rows, d, out, s);
  }
}

}  // namespace hbl
