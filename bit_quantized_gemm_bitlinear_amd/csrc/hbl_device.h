// hbl_device.h — device helpers shared by the HIP kernels of libhbl (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hbl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes from `base` (stride 0, raw 32-bit offsets; offsets past
// the end read zeros).
__device__ __forceinline__ v4u_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return v4u_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// One 16-byte-per-lane load from global memory into LDS (buffer_load_dwordx4 ... lds): lane
// l's bytes at rsrc base + voff + soff land at LDS byte lds_base + 16 l.  Written as inline
// assembly: the compiler's own form makes every later LDS read wait for all loads of this kind
// in flight (it cannot tell which LDS bytes they write), which would drain a load pipeline at
// every step.  A kernel using it therefore waits for these loads itself (s_waitcnt vmcnt; they
// complete in issue order), and the memory clobber keeps the compiler from moving LDS reads
// across them.  M0 holds the LDS base (wave-uniform); one
// wait state separates its write from the load that reads it.  M0 is a register the compiler
// reserves: it keeps no value there across this statement in these kernels (it sets M0 only
// for instructions they do not use), so clobbering it is safe here and its warning is silenced.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(v4u_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// bf16 bit patterns live in the top half of an fp32 word; the conversion is exact.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bit pattern, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Two fp32 bit patterns -> two bf16 in one word (lo first), round to nearest even, by the
// packed conversion instruction (v_cvt_pk_bf16_f32).  For every non-NaN input, denormals
// included (the kernels run with fp32 denormals preserved), the bits are those of
// f32_to_bf16_rne.
__device__ __forceinline__ uint32_t bf16x2_rne(uint32_t lo, uint32_t hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  const bf16x2v_t b = __builtin_convertvector(f32x2_t{__uint_as_float(lo), __uint_as_float(hi)}, bf16x2v_t);
  return __builtin_bit_cast(uint32_t, b);
}

// e^x for the SwiGLU gate, in a few instructions: x log2(e) = n + r with n an integer and
// |r| <= 1/2, where log2(e) is split into its fp32 value and the remainder so that r carries
// only its own rounding; 2^r comes from v_exp_f32 and n is added to the exponent
// (v_ldexp_f32, which gives 0 or inf past the fp32 range).  x is clamped to +-150 first, far
// outside that range, so that the reduction never sees an infinity.
__device__ __forceinline__ float exp_gate(float x) {
  const float l2e_hi = 1.44269502162933349609375f;  // fp32 nearest to log2(e)
  const float l2e_lo = 1.9259629911e-8f;            // log2(e) - l2e_hi
  x = __builtin_fminf(__builtin_fmaxf(x, -150.0f), 150.0f);
  const float n = __builtin_rintf(x * l2e_hi);
  const float r = __builtin_fmaf(x, l2e_hi, -n) + x * l2e_lo;
  return __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(r), (int)n);
}

// SwiGLU gate: silu(g) * u with silu(v) = v / (1 + exp(-v)) = v * rcp(1 + exp(-v)), in fp32
// with exp_gate and v_rcp_f32 (each about an ulp).  Shared by the standalone kernel and the
// fused GEMM epilogue so both give the same bits.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float sg = g * __builtin_amdgcn_rcpf(1.0f + exp_gate(-g));
  return sg * u;
}

// Round half to even then convert (v_rndne_f32 + v_cvt_i32_f32).
__device__ __forceinline__ int rne_int(float v) { return (int)__builtin_rintf(v); }

// Eight consecutive INT4 codes c[0..7] (k = 8h + 0..7 of a 16-code group) -> one 32-bit
// word of the packed INT4 layout: byte i holds c[i] (low nibble) and c[i+4] (high nibble).
__device__ __forceinline__ uint32_t pack8_a4(int c0, int c1, int c2, int c3, int c4, int c5, int c6,
                                             int c7) {
  uint32_t b0 = (uint32_t)(c0 & 15) | ((uint32_t)(c4 & 15) << 4);
  uint32_t b1 = (uint32_t)(c1 & 15) | ((uint32_t)(c5 & 15) << 4);
  uint32_t b2 = (uint32_t)(c2 & 15) | ((uint32_t)(c6 & 15) << 4);
  uint32_t b3 = (uint32_t)(c3 & 15) | ((uint32_t)(c7 & 15) << 4);
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Four consecutive INT8 codes -> one little-endian word.
__device__ __forceinline__ uint32_t pack4_a8(int c0, int c1, int c2, int c3) {
  return (uint32_t)(c0 & 255) | ((uint32_t)(c1 & 255) << 8) | ((uint32_t)(c2 & 255) << 16) |
         ((uint32_t)(c3 & 255) << 24);
}

// Butterfly reductions across the lanes of a wave (width = power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int WIDTH>
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace hbl
