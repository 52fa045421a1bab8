// actquant_store.h — quantisation and packed stores of activation codes, shared by the
// activation kernels (k_actquant.hip, k_actquant_mfma.hip).  Formats are those of hbl.h.
#pragma once
#include "hbl_device.h"

namespace hbl {
namespace {

// ABITS: 4 = INT4 codes packed as nibbles, 8 = INT8 codes, 6 = INT4 codes (Qb = 7) stored as
// FP6 E2M3 (6 bits each, code k at bits [6k, 6k+6) of the row's little-endian bit string),
// 5 = INT4 codes packed as nibbles with the absmean statistic instead of absmax:
// b = mean|z| (fp64 sum), s = fl32(1/b), q = clamp(rint(z*s), -8, 7), deq = b*r*hK.
template <int ABITS>
struct QB {
  static constexpr float value = ABITS == 8 ? 127.0f : 7.0f;
};

template <int ABITS>
constexpr int row_bytes(int K) { return (ABITS == 4 || ABITS == 5) ? K / 2 : (ABITS == 8 ? K : K * 6 / 8); }

typedef float v16f_t __attribute__((ext_vector_type(16)));

// 2 to 32 integer-valued floats (|q| <= 7) -> FP6 E2M3, packed 6 bits each in element order.
// The hardware conversion interleaves its two 16-wide operands (element 2i from the first,
// 2i+1 from the second); the scale 1.0 leaves values unscaled.  Exact for these integers.
template <int NV>
__device__ __forceinline__ void fp6_pack(const float* q, uint32_t (&w)[6]) {
  v16f_t ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = 2 * i < NV ? q[2 * i] : 0.0f;
    od[i] = 2 * i + 1 < NV ? q[2 * i + 1] : 0.0f;
  }
  const auto r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
#pragma unroll
  for (int i = 0; i < 6; ++i) w[i] = (uint32_t)r[i];
}

// Store NWORDS packed 32-bit words to dst (aligned to 4 * min(NWORDS, 4) bytes).
template <int NWORDS>
__device__ __forceinline__ void store_words(uint8_t* dst, const uint32_t* w) {
  if constexpr (NWORDS >= 4) {
#pragma unroll
    for (int d = 0; d < NWORDS; d += 4)
      *reinterpret_cast<uint4*>(dst + 4 * d) = make_uint4(w[d], w[d + 1], w[d + 2], w[d + 3]);
  } else if constexpr (NWORDS == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
    *reinterpret_cast<uint32_t*>(dst) = w[0];
  }
}

// Round-half-even to an integer through the fp32 adder: for |v| <= 2^21, v + (1.5*2^23 + c)
// rounds to the integer rint(v) + c (spacing 1 in [2^23, 2^24), ties to even; c even keeps
// the parity), whose low mantissa bits are then rint(v) + c in two's complement.
__device__ __forceinline__ uint32_t rne_bits(float v, float magic) { return __float_as_uint(v + magic); }

// Quantise a run of RL consecutive row elements v[0 .. RL) (scale s) starting at row
// element k0 and store its packed bytes.
//  INT4: offset magic +8 gives low nibble q+8 in [1,15] with zero bits above it, so a pair
//        (lo, hi) becomes one byte with a single shift-or; four bytes are gathered with
//        v_perm and the offset is removed with one xor (q+8 ^ 8 = q mod 16).
//  INT8: the low byte of the rounded value is q mod 256; four are gathered with v_perm.
template <int ABITS, int RL>
__device__ __forceinline__ void store_run(const float* v, float s, uint8_t* __restrict__ crow, int k0) {
  constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
  if constexpr (ABITS == 6) {
    // rint first (the FP6 grid is finer than the integers below 4), then the exact conversion.
    uint8_t* dst = crow + (k0 / 8) * 6;
#pragma unroll
    for (int c = 0; c < RL; c += 32) {
      constexpr int NV = RL < 32 ? RL : 32;
      float q[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) q[i] = __builtin_rintf(v[c + i] * s) + 0.0f;  // +0.0f: -0 -> +0 (code 0x00)
      uint32_t w[6];
      fp6_pack<NV>(q, w);
      if constexpr (NV == 32) {
#pragma unroll
        for (int i = 0; i < 3; ++i) reinterpret_cast<uint2*>(dst + 24 * (c / 32))[i] = make_uint2(w[2 * i], w[2 * i + 1]);
      } else if constexpr (NV == 16) {
#pragma unroll
        for (int i = 0; i < 3; ++i) reinterpret_cast<uint32_t*>(dst)[i] = w[i];
      } else {  // 8 codes = 48 bits, 2-byte aligned
        uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
        d16[0] = (uint16_t)(w[0] & 0xffffu);
        d16[1] = (uint16_t)(w[0] >> 16);
        d16[2] = (uint16_t)(w[1] & 0xffffu);
      }
    }
  } else if constexpr (ABITS == 4 || ABITS == 5) {
    // absmean codes can exceed the INT4 range: clamp before rounding (same as after, the
    // bounds being integers)
    auto sc = [&](float z) { return ABITS == 5 ? fminf(fmaxf(z * s, -8.0f), 7.0f) : z * s; };
    uint32_t w[RL / 8];
#pragma unroll
    for (int d = 0; d < RL / 8; ++d) {
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = rne_bits(sc(v[8 * d + i]), MAGIC + 8.0f);
        const uint32_t hi = rne_bits(sc(v[8 * d + i + 4]), MAGIC + 8.0f);
        b[i] = (hi << 4) | lo;  // byte 0 = (hi+8) << 4 | (lo+8); higher bytes unused
      }
      const uint32_t b01 = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
      const uint32_t b23 = __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
      w[d] = (b01 | b23) ^ 0x88888888u;
    }
    store_words<RL / 8>(crow + k0 / 2, w);
  } else {
    uint32_t w[RL / 4];
#pragma unroll
    for (int d = 0; d < RL / 4; ++d) {
      const uint32_t q0 = rne_bits(v[4 * d + 0] * s, MAGIC), q1 = rne_bits(v[4 * d + 1] * s, MAGIC);
      const uint32_t q2 = rne_bits(v[4 * d + 2] * s, MAGIC), q3 = rne_bits(v[4 * d + 3] * s, MAGIC);
      const uint32_t lo = __builtin_amdgcn_perm(q1, q0, 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(q3, q2, 0x04000c0cu);
      w[d] = lo | hi;
    }
    store_words<RL / 4>(crow + k0, w);
  }
}

}  // namespace
}  // namespace hbl
