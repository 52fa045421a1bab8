// actquant_mfma.h — the online Hadamard transform of bf16 activation rows with five or six of
// its butterfly stages on the matrix cores, shared by the activation kernel (k_actquant_mfma.hip)
// and the fused decode kernel (k_actquant.hip).
//
// BitNet v2 write-up, section H-BitLinear模塊: the activations are normalised and then
// transformed by an online Hadamard transform, computed with the fast Hadamard transform in
// O(n log n), before the per-token quantisation.
//
// The Sylvester matrix factors over the index bits: H_K is the product, over the bits b of
// the element index, of a 2-point butterfly on b, and these factors commute.  Five bits can
// therefore be transformed at once by a product with H_32 (entries +-1, exact in bf16): the
// raw bf16 values are the A operand of v_mfma_f32_32x32x16_bf16 and H_32 the B operand, so
// every product is exact and the sums are accumulated in fp32 by the matrix core.  The other
// index bits are transformed by fp32 butterflies in registers, around one transpose through
// LDS.  Stage order and summation order differ from the plain in-place loop, so z agrees with
// it up to fp32 rounding; on integer-valued rows whose transform stays below 2^24 every sum
// is exact and z is identical.  Where the next index bit (e10) also indexes the row, its
// butterfly is folded into the products too (hm_front).
//
// Layout.  A block of 4 waves transforms a slab of 16384 consecutive elements (16384 / K rows
// of K = 2^L elements, 10 <= L <= 14); element E of the slab has index bits e0..e13 and
// e0..e(L-1) index the row.
//   raw load: wave w, lane l, chunk c (16 bytes = 8 bf16): E = 4096 w + 512 c + 8 l + (0..7)
//   product p (chunks 2p, 2p+1): A rows i = e3..e7 (lanes 0..31), k = e0..e2 (the 8 values of
//     a lane), e8 (lane half) and e9 (chunk parity).  Result lane l holds column j = l % 32,
//     the transformed bits (e0, e1, e2, e8, e9), and 16 rows i: register bits e3, e4, e6, e7,
//     lane bit 5 = e5, and p = (e10, e11)
//   e10 on the matrix cores where it indexes the row (the products then hold z's e10 bit in
//     the place of p's)
//   register stages: e3, e4, e6, e7, then e11 where it indexes the row
//   LDS transpose; registers then hold runs of consecutive elements (e0, e1, e2, ...) and the
//   bits still to transform, e5 and (for L = 13, 14) e12, e13; stages on them.
#pragma once
#include "hbl_device.h"

namespace hbl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int HM_SLAB = 16384;   // elements per slab: 4 waves x 8 chunks x 512
constexpr int HM_WG = 256;

// LDS address (in floats) of slab element E: 4 floats of padding per 64 elements and 8 more
// per 512.  The padding is linear in disjoint index bits, so every register's offset is an
// immediate; groups of 4 consecutive elements stay contiguous; and in a 32-bank model both
// sides of the transpose are free of conflicts (the b32 stores of the matrix-core layout and
// the b128 loads of runs).
__host__ __device__ constexpr int hm_lds(int E) { return E + 4 * (E >> 6) + 8 * (E >> 9); }
constexpr int HM_LDS_FLOATS = hm_lds(HM_SLAB - 1) + 1;

// Matrix-core layout: element bits of lane l and of register reg = 16 p + r.
__device__ __forceinline__ int hm_pre_lane(int l) {
  return (l & 7) | (((l >> 3) & 1) << 8) | (((l >> 4) & 1) << 9) | (((l >> 5) & 1) << 5);
}
__host__ __device__ constexpr int hm_pre_reg(int reg) {
  return ((reg & 1) << 3) | (((reg >> 1) & 1) << 4) | (((reg >> 2) & 1) << 6) | (((reg >> 3) & 1) << 7) |
         (((reg >> 4) & 1) << 10) | (((reg >> 5) & 1) << 11);
}

// Layout after the transpose: register bits j0..j5, lane bits l0..l5, wave bits w0, w1.
template <int L>
struct HmPost {
  // element bit of register bit i / lane bit i / wave bit i
  static constexpr int rb(int i) {
    return L == 14 ? (i < 3 ? i : (i == 3 ? 5 : (i == 4 ? 12 : 13)))
                   : (L == 13 ? (i < 4 ? i : (i == 4 ? 5 : 12)) : i);
  }
  static constexpr int lb(int i) {
    return L == 14 ? (i < 2 ? 3 + i : 4 + i) : (L == 13 ? (i == 0 ? 4 : 5 + i) : 6 + i);
  }
  static constexpr int wb(int i) { return L == 14 ? 10 + i : (L == 13 ? (i == 0 ? 11 : 13) : 12 + i); }
  static constexpr int reg_E(int j) {
    int e = 0;
    for (int i = 0; i < 6; ++i) e |= ((j >> i) & 1) << rb(i);
    return e;
  }
  static __device__ __forceinline__ int thread_E(int w, int l) {
    int e = 0;
#pragma unroll
    for (int i = 0; i < 6; ++i) e |= ((l >> i) & 1) << lb(i);
#pragma unroll
    for (int i = 0; i < 2; ++i) e |= ((w >> i) & 1) << wb(i);
    return e;
  }
  // runs of consecutive elements in registers: register bits 0 .. RUNB-1 are e0 .. e(RUNB-1)
  static constexpr int RUNB = L == 14 ? 3 : (L == 13 ? 4 : 6);
  static constexpr int RL = 1 << RUNB;
  // register bits still to transform after the transpose: e5, and e12, e13 below L
  static constexpr int NSTAGE = L == 14 ? 3 : (L == 13 ? 2 : 1);
  static constexpr int stage_bit(int s) { return L == 14 ? 3 + s : (L == 13 ? 4 + s : 5); }
  // lanes of a wave that share a row, and waves that share a row
  static constexpr int ROW_LANES = L >= 12 ? 64 : (L == 11 ? 32 : 16);
  static constexpr int ROW_WAVES = L >= 12 ? (1 << (L - 12)) : 1;
};

// Butterfly on register bit B of 64 values: (a, b) -> (a + b, a - b).
template <int B>
__device__ __forceinline__ void hm_stage(float (&v)[64]) {
  constexpr int h = 1 << B;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    if ((j & h) == 0) {
      const float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
}

// H_32 as this lane's B operand for k-step s: B[k][j] = (-1)^popcount(k & j) with k bits
// (e0, e1, e2) = item, e8 = lane half, e9 = s, and j = lane % 32 with bits (e0, e1, e2, e8, e9).
__device__ __forceinline__ bf16x8_t hm_hadamard_b(int lane, int s) {
  const int j = lane & 31;
  const int kh = lane >> 5;
  bf16x8_t b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int par = __builtin_popcount(e & j) + (kh & (j >> 3)) + (s & (j >> 4));
    b[e] = (par & 1) ? (__bf16)-1.0f : (__bf16)1.0f;
  }
  return b;
}

// Reductions over WIDTH = 16, 32 or 64 lanes: DPP exchanges inside each row of 16 lanes (pair,
// quad, half-row and row mirrors), then the row results read into scalars and combined, so no
// LDS round trip is needed.  Every lane of a WIDTH group ends with the same value, in a fixed
// order of operations.
template <int CTRL>
__device__ __forceinline__ uint32_t hm_dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int WIDTH>
__device__ __forceinline__ float hm_wave_max(float v, int lane) {
  v = __builtin_fmaxf(v, __uint_as_float(hm_dpp<DPP_XOR1>(__float_as_uint(v))));
  v = __builtin_fmaxf(v, __uint_as_float(hm_dpp<DPP_XOR2>(__float_as_uint(v))));
  v = __builtin_fmaxf(v, __uint_as_float(hm_dpp<DPP_HALF_MIRROR>(__float_as_uint(v))));
  v = __builtin_fmaxf(v, __uint_as_float(hm_dpp<DPP_MIRROR>(__float_as_uint(v))));
  if constexpr (WIDTH == 16) return v;
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  if constexpr (WIDTH == 32) return lane < 32 ? __builtin_fmaxf(r0, r1) : __builtin_fmaxf(r2, r3);
  return __builtin_fmaxf(__builtin_fmaxf(r0, r1), __builtin_fmaxf(r2, r3));
}

__device__ __forceinline__ double hm_dpp_d(double v, int step) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  switch (step) {
    case 0: lo = hm_dpp<DPP_XOR1>(lo); hi = hm_dpp<DPP_XOR1>(hi); break;
    case 1: lo = hm_dpp<DPP_XOR2>(lo); hi = hm_dpp<DPP_XOR2>(hi); break;
    case 2: lo = hm_dpp<DPP_HALF_MIRROR>(lo); hi = hm_dpp<DPP_HALF_MIRROR>(hi); break;
    default: lo = hm_dpp<DPP_MIRROR>(lo); hi = hm_dpp<DPP_MIRROR>(hi); break;
  }
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double hm_readlane_d(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int WIDTH>
__device__ __forceinline__ double hm_wave_sum(double v, int lane) {
#pragma unroll
  for (int st = 0; st < 4; ++st) v += hm_dpp_d(v, st);
  if constexpr (WIDTH == 16) return v;
  const double r0 = hm_readlane_d(v, 0), r1 = hm_readlane_d(v, 16);
  const double r2 = hm_readlane_d(v, 32), r3 = hm_readlane_d(v, 48);
  if constexpr (WIDTH == 32) return lane < 32 ? r0 + r1 : r2 + r3;
  return (r0 + r1) + (r2 + r3);
}

// The slab's raw chunks of this thread (raw layout) for rows slab*R + (E >> L) of x [M, K],
// rows past M taken from row M-1 (computed, never stored).
template <int L>
__device__ __forceinline__ void hm_load(uint4 (&raw)[8], const uint16_t* __restrict__ x, int64_t M, int64_t slab,
                                        int w, int lane) {
  constexpr int K = 1 << L;
  constexpr int R = HM_SLAB / K;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int E = 4096 * w + 512 * c + 8 * lane;
    int64_t row = slab * R + (E >> L);
    row = row < M ? row : M - 1;
    // nontemporal: x is read once, so its lines need not displace anything in the caches
    // (2 % faster than plain loads at the 7B Wdown shape)
    const v4u_t t = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(x + row * K + (E & (K - 1))));
    raw[c] = uint4{t.x, t.y, t.z, t.w};
  }
}

// Row statistics of one slab, for this thread's row in the layout after the transpose.
struct HmStats {
  float amax;    // max |z| (absmax statistic)
  double sabs;   // sum |z| (absmean statistic, ABITS 5)
  double ss;     // sum of x^2 (RMSNorm)
};

// Transform bits taken by the matrix cores: the five of the product with H_32, plus e10 where it
// indexes the row (a product with H_64).
template <int L>
__device__ __forceinline__ constexpr int hm_mfma_bits() {
  return L >= 11 ? 6 : 5;
}

// Front of the transform of the slab held in raw: the partial sums of squares (NM != 0) and the
// products on the matrix cores, written to v in the matrix-core layout.  Nothing here touches
// LDS, and raw may be reloaded as soon as this returns.
//
// Chunks 2p and 2p + 1 hold, for each of the 32 A rows, 32 values whose transform bits are
// (e0, e1, e2, e8, e9): t_p = A_2p H_32[0:16] + A_2p+1 H_32[16:32] is their 32-point transform,
// and the two bits of p are e10 and e11.  Where e10 indexes the row its 2-point butterfly is
// folded into the products as well: the accumulator of one product is the C input of the next,
// so t_2g + t_2g+1 and t_2g - t_2g+1 both continue from t_2g, the second with H negated (six
// products per pair of p instead of four products and a butterfly stage).  Every product is
// exact and the sums are fp32 sums of the matrix core, so z agrees with the butterfly order up
// to fp32 rounding, and exactly on the integer class.
template <int L, int NM>
__device__ __forceinline__ void hm_front(const uint4 (&raw)[8], const bf16x8_t hb0, const bf16x8_t hb1,
                                         float (&v)[64], float (&ssp)[4]) {
  // ---- sums of squares on the raw bf16 (squares exact; fp32 sums per pair of chunks) ----
#pragma unroll
  for (int i = 0; i < 4; ++i) ssp[i] = 0.0f;
  if constexpr (NM != 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t d[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2_t b = __builtin_bit_cast(bf16x2_t, d[q]);
        ssp[c >> 1] = __builtin_amdgcn_fdot2_f32_bf16(b, b, ssp[c >> 1], false);
      }
    }
  }

  // ---- products on the matrix cores ----
  constexpr int MB = hm_mfma_bits<L>();
  const bf16x8_t nb0 = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(v4u_t, hb0) ^ 0x80008000u);
  const bf16x8_t nb1 = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(v4u_t, hb1) ^ 0x80008000u);
  // C + A_c H (H negated if neg), H's half chosen by the chunk parity e9
  auto mma = [&](int c, bool neg, f32x16_t acc) __attribute__((always_inline)) {
    const bf16x8_t b = (c & 1) ? (neg ? nb1 : hb1) : (neg ? nb0 : hb0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, raw[c]), b, acc, 0, 0, 0);
  };
  auto put = [&](int p, const f32x16_t& d) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) v[16 * p + r] = d[r];
  };
  if constexpr (MB == 5) {
#pragma unroll
    for (int p = 0; p < 4; ++p) put(p, mma(2 * p + 1, false, mma(2 * p, false, f32x16_t{})));
  } else {
    static_assert(MB == 6, "five or six bits on the matrix cores");
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const f32x16_t t = mma(4 * g + 1, false, mma(4 * g, false, f32x16_t{}));
      put(2 * g, mma(4 * g + 3, false, mma(4 * g + 2, false, t)));
      put(2 * g + 1, mma(4 * g + 3, true, mma(4 * g + 2, true, t)));
    }
  }
}

// Back of the transform: on entry v holds the products of hm_front and ssp its partial sums of
// squares; on return v holds this thread's 64 values of z in the layout after the transpose
// and st its row's statistics.
// Synchronisation: for L <= 12 a row lives in one wave and the wave's LDS region is its own,
// so no block barrier is needed (LDS instructions of a wave execute in order).  For L >= 13 a
// row spans 2 or 4 waves: one block barrier after the transpose stores, one after the partial
// statistics are written.  Consecutive calls need no barrier between them: every wave reads
// this slab's LDS and reduction slots before it reaches the second barrier, and writes the
// next slab's slots only after the next call's first barrier.
template <int L, int ABITS, int NM>
__device__ __forceinline__ void hm_back(float* __restrict__ lds, float* redf, double* redd, double* redd2, int w,
                                        int lane, float (&v)[64], const float (&ssp)[4], HmStats& st) {
  using P = HmPost<L>;
  constexpr int MB = hm_mfma_bits<L>();
  // ---- register stages: e3, e4, e6, e7, then e10 (unless the matrix cores took it) and e11
  // where they index the row ----
  hm_stage<0>(v);
  hm_stage<1>(v);
  hm_stage<2>(v);
  hm_stage<3>(v);
  if constexpr (L >= 11 && MB < 6) hm_stage<4>(v);
  if constexpr (L >= 12) hm_stage<5>(v);

  // ---- transpose through LDS ----
  {
    float* base = lds + hm_lds(4096 * w + hm_pre_lane(lane));
#pragma unroll
    for (int reg = 0; reg < 64; ++reg) base[hm_lds(hm_pre_reg(reg))] = v[reg];
  }
  if constexpr (L >= 13) {
    __syncthreads();
  } else {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  {
    const float* base = lds + hm_lds(P::thread_E(w, lane));
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
      const float4 q = *reinterpret_cast<const float4*>(base + hm_lds(P::reg_E(j)));
      v[j] = q.x;
      v[j + 1] = q.y;
      v[j + 2] = q.z;
      v[j + 3] = q.w;
    }
  }
  // ---- the remaining stages: e5, then e12, e13 where they index the row ----
  hm_stage<P::stage_bit(0)>(v);
  if constexpr (P::NSTAGE > 1) hm_stage<P::stage_bit(1)>(v);
  if constexpr (P::NSTAGE > 2) hm_stage<P::stage_bit(2)>(v);

  // ---- per-row statistics ----
  // Rows in the raw layout: the row of a thread's chunks is wave-uniform for L >= 12 and
  // given by the chunk pair for L < 12 (e11 = c2, e10 = c1); in the layout after the
  // transpose it is wave-uniform for L >= 12 and given by lane bits for L < 12 (e11 = lane
  // bit 5, e10 = lane bit 4).  Waves keep their row bits across the transpose.
  st.ss = 0.0;
  if constexpr (NM != 0) {
    double s_row[4] = {0.0, 0.0, 0.0, 0.0};
    constexpr int NR = L >= 12 ? 1 : (L == 11 ? 2 : 4);
    if constexpr (L >= 12) {
      s_row[0] = (double)ssp[0] + (double)ssp[1] + (double)ssp[2] + (double)ssp[3];
    } else if constexpr (L == 11) {
      s_row[0] = (double)ssp[0] + (double)ssp[1];
      s_row[1] = (double)ssp[2] + (double)ssp[3];
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) s_row[p] = (double)ssp[p];
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) s_row[i] = hm_wave_sum<64>(s_row[i], lane);
    if constexpr (L >= 13) {
      if (lane == 0) redd[w] = s_row[0];
    } else if constexpr (L == 12) {
      st.ss = s_row[0];
    } else if constexpr (L == 11) {
      st.ss = (lane >> 5) ? s_row[1] : s_row[0];
    } else {
      const int rq = (lane >> 4) & 3;
      st.ss = rq == 0 ? s_row[0] : (rq == 1 ? s_row[1] : (rq == 2 ? s_row[2] : s_row[3]));
    }
  }
  st.amax = 0.0f;
  st.sabs = 0.0;
  if constexpr (ABITS == 5) {
    double sa = 0.0;
#pragma unroll
    for (int j = 0; j < 64; ++j) sa += (double)fabsf(v[j]);
    st.sabs = hm_wave_sum<P::ROW_LANES>(sa, lane);
    if constexpr (L >= 13) {
      if (lane == 0) redd2[w] = st.sabs;
    }
  } else {
    // four chains of v_max3 (two new values each)
    float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 64; j += 8) {
#pragma unroll
      for (int c = 0; c < 4; ++c) m[c] = __builtin_fmaxf(__builtin_fmaxf(m[c], fabsf(v[j + 2 * c])), fabsf(v[j + 2 * c + 1]));
    }
    st.amax = hm_wave_max<P::ROW_LANES>(__builtin_fmaxf(__builtin_fmaxf(m[0], m[1]), __builtin_fmaxf(m[2], m[3])), lane);
    if constexpr (L >= 13) {
      if (lane == 0) redf[w] = st.amax;
    }
  }
  if constexpr (L >= 13) {
    __syncthreads();
    // waves of a row: all four (L = 14) or the pair sharing e13 = wave bit 1 (L = 13), in
    // both layouts
    const int w0 = L == 14 ? 0 : (w & 2);
    if constexpr (NM != 0) {
      st.ss = redd[w0];
#pragma unroll
      for (int i = 1; i < P::ROW_WAVES; ++i) st.ss += redd[w0 + i];
    }
    if constexpr (ABITS == 5) {
      st.sabs = redd2[w0];
#pragma unroll
      for (int i = 1; i < P::ROW_WAVES; ++i) st.sabs += redd2[w0 + i];
    } else {
      st.amax = redf[w0];
#pragma unroll
      for (int i = 1; i < P::ROW_WAVES; ++i) st.amax = __builtin_fmaxf(st.amax, redf[w0 + i]);
    }
  }
}

// The whole transform of the slab held in raw; `after_mfma` runs once the matrix cores have
// read raw (the caller may reload it there).
template <int L, int ABITS, int NM, typename AfterMfma>
__device__ __forceinline__ void hm_transform(uint4 (&raw)[8], const bf16x8_t hb0, const bf16x8_t hb1,
                                             float* __restrict__ lds, float* redf, double* redd, double* redd2,
                                             int w, int lane, float (&v)[64], HmStats& st, AfterMfma&& after_mfma) {
  float ssp[4];
  hm_front<L, NM>(raw, hb0, hb1, v, ssp);
  after_mfma();
  hm_back<L, ABITS, NM>(lds, redf, redd, redd2, w, lane, v, ssp, st);
}

}  // namespace
}  // namespace hbl
