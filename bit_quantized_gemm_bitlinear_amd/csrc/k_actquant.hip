// k_actquant.hip — fused per-token activation path of H-BitLinear:
//   load (bf16/fp32) -> RMSNorm statistics -> online fast Walsh-Hadamard transform ->
//   per-token absmax -> INT4/INT8 codes -> packed store + one dequant factor per row.
//
// BitNet v2 write-up, section H-BitLinear模塊: before the activations are quantised the
// layer applies LN and an online Hadamard transform computed with the fast Hadamard
// transform (O(n log n)); the transform reshapes the outlier-heavy inputs of Wo / Wdown
// into a Gaussian-like distribution; the activations are then quantised per token to INT8
// or INT4.  bitnet.cpp article, section "6 页论文，引入 1 bit LLM": activations are scaled
// into [-Qb, Qb] without a zero point.
//
// Transform (use_hadamard = 1, K = 2^L, 6 <= L <= 15).  Every thread owns 64 values of one
// row.  The butterfly stages run strictly in ascending order of the index bit they act on
// (h = 1, 2, 4, ..., K/2), so the fp32 result is bit-identical to the plain in-place loop.
// A stage always acts on a register bit of the current layout; between groups of stages the
// row is transposed through LDS so that the next index bits become register bits:
//   phase 0: registers = index bits 0..5 (64 consecutive elements, loaded from HBM)
//   later phases: registers = the next active index bits + the lowest index bits, so the
//   last phase leaves runs of >= 8 consecutive elements in registers, ready to be packed
//   and stored without another transpose.
// LDS rows are padded with 4 floats every 64 (the padded address is linear in disjoint
// index bits, so every register offset is a compile-time immediate).
//
// The RMSNorm factor r and 1/sqrt(K) are not applied to the values: absmax codes do not
// change under a positive per-row scale, so both are folded into deq.
#include <cmath>

#include "actquant_mfma.h"
#include "actquant_store.h"
#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

struct PhaseDesc {
  int lo;  // first active index bit
  int a;   // number of active index bits (butterfly stages) in this phase
};

constexpr int nphases(int L) { return L <= 6 ? 1 : (L <= 9 ? 2 : 3); }

constexpr PhaseDesc phase_desc(int L, int p) {
  if (p == 0) return PhaseDesc{0, L < 6 ? L : 6};
  if (L <= 9) return PhaseDesc{6, L - 6};
  if (L <= 12) return p == 1 ? PhaseDesc{6, L - 9} : PhaseDesc{L - 3, 3};
  return p == 1 ? PhaseDesc{6, 6} : PhaseDesc{12, L - 12};
}

// Register j of a thread in phase P holds row element  base(t) + off(j):
//   j's low c = 6-a bits -> index bits 0..c-1 ; j's high a bits -> index bits lo..lo+a-1;
//   the thread index t fills the remaining index bits in ascending order.
template <int L, int P>
struct Layout {
  static constexpr PhaseDesc d = phase_desc(L, P);
  static constexpr int a = d.a;
  static constexpr int lo = d.lo;
  static constexpr int c = 6 - d.a;
  static __device__ __forceinline__ constexpr int off(int j) {
    return (j & ((1 << c) - 1)) | ((j >> c) << lo);
  }
  static __device__ __forceinline__ int base(int t) {
    return ((t & ((1 << (lo - c)) - 1)) << c) | ((t >> (lo - c)) << (lo + a));
  }
};

__device__ __forceinline__ constexpr int padded(int i) { return i + ((i >> 6) << 2); }

// Butterfly stages on register bits [c, c + a) in ascending order.
template <int C, int A>
__device__ __forceinline__ void stages(float (&v)[64]) {
#pragma unroll
  for (int s = 0; s < A; ++s) {
    const int h = 1 << (C + s);
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      if ((j & h) == 0) {
        float x0 = v[j], x1 = v[j + h];
        v[j] = x0 + x1;
        v[j + h] = x0 - x1;
      }
    }
  }
}

// Row-wide reductions for rows spread over T threads (T a power of two).  Threads of a
// row are contiguous in the block; rows of <= 64 threads stay inside one wave.
template <int T>
__device__ __forceinline__ float row_max(float v, float* red) {
  if constexpr (T <= 64) {
    return wave_max<T>(v);
  } else {
    v = wave_max<64>(v);
    const int tid = threadIdx.x;
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    const int w0 = (tid / T) * (T / 64);
    float m = red[w0];
#pragma unroll
    for (int i = 1; i < T / 64; ++i) m = fmaxf(m, red[w0 + i]);
    return m;
  }
}

template <int T>
__device__ __forceinline__ double row_sum(double v, double* red) {
  if constexpr (T <= 64) {
    return wave_sum<T>(v);
  } else {
    v = wave_sum<64>(v);
    const int tid = threadIdx.x;
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    const int w0 = (tid / T) * (T / 64);
    double s = red[w0];
#pragma unroll
    for (int i = 1; i < T / 64; ++i) s += red[w0 + i];
    return s;
  }
}

template <int L, int P, int ROWF>
__device__ __forceinline__ void lds_read(float (&v)[64], const float* rowlds, int t) {
  using LY = Layout<L, P>;
  const float* b = rowlds + padded(LY::base(t));
#pragma unroll
  for (int j = 0; j < 64; ++j) v[j] = b[padded(LY::off(j))];
}

template <int L, int P, int ROWF>
__device__ __forceinline__ void lds_write(const float (&v)[64], float* rowlds, int t) {
  using LY = Layout<L, P>;
  float* b = rowlds + padded(LY::base(t));
#pragma unroll
  for (int j = 0; j < 64; ++j) b[padded(LY::off(j))] = v[j];
}

template <int L>
constexpr int block_threads() {
  return (1 << L) / 64 > 256 ? (1 << L) / 64 : 256;
}

// Raw input of one thread's 64 consecutive row elements (bf16: 8 x 16 bytes, fp32: 16 x 16).
template <int XT>
struct RowChunk {
  uint4 w[XT == 1 ? 8 : 16];
};

template <int XT>
__device__ __forceinline__ void load_chunk(RowChunk<XT>& c, const void* x, int64_t elem0) {
  const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(x) + elem0 * (XT == 1 ? 2 : 4));
#pragma unroll
  for (int i = 0; i < (XT == 1 ? 8 : 16); ++i) c.w[i] = src[i];
}

// The same 64 elements taken as 8 chunks of 8 consecutive ones, chunk i at elem0 + 8*T*i:
// the T threads of a row then read it in fully coalesced 16-byte units.
template <int XT, int T>
__device__ __forceinline__ void load_chunk_strided(RowChunk<XT>& c, const void* x, int64_t elem0) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (XT == 1) {
      c.w[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + elem0 + 8 * T * i);
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + elem0 + 8 * T * i);
      c.w[2 * i] = p[0];
      c.w[2 * i + 1] = p[1];
    }
  }
}

template <int XT>
__device__ __forceinline__ void unpack_chunk(const RowChunk<XT>& c, float (&v)[64]) {
#pragma unroll
  for (int i = 0; i < (XT == 1 ? 8 : 16); ++i) {
    const uint4 w = c.w[i];
    if constexpr (XT == 1) {
      v[8 * i + 0] = bf16lo(w.x);
      v[8 * i + 1] = bf16hi(w.x);
      v[8 * i + 2] = bf16lo(w.y);
      v[8 * i + 3] = bf16hi(w.y);
      v[8 * i + 4] = bf16lo(w.z);
      v[8 * i + 5] = bf16hi(w.z);
      v[8 * i + 6] = bf16lo(w.w);
      v[8 * i + 7] = bf16hi(w.w);
    } else {
      v[4 * i + 0] = __uint_as_float(w.x);
      v[4 * i + 1] = __uint_as_float(w.y);
      v[4 * i + 2] = __uint_as_float(w.z);
      v[4 * i + 3] = __uint_as_float(w.w);
    }
  }
}

// NM: 0 = no norm, 1 = RMSNorm with unit gamma, 2 = RMSNorm with gamma.
// Blocks are persistent: block b handles row groups b, b + gridDim.x, ...; the raw input of
// the next group is loaded into registers while the current one is transformed.
// HT = false skips the transform (the BitLinear path for K = 2^L): each thread then holds 8
// chunks of 8 consecutive elements, chunk i at row offset 8 (t + T i), so that loads and code
// stores are coalesced across the row's threads, and quantises them with no LDS exchange.
template <int L, int ABITS, int XT, int NM, bool HT>
__device__ __forceinline__ void actquant_rows(
    const void* __restrict__ x, int64_t M, const float* __restrict__ gamma, float eps, float hK,
    uint8_t* __restrict__ codes, float* __restrict__ deq) {
  constexpr int K = 1 << L;
  constexpr int T = K / 64;           // threads per row
  constexpr int WG = block_threads<L>();
  constexpr int R = WG / T;           // rows per block
  constexpr int NP = HT ? nphases(L) : 1;
  constexpr int ROWF = K + K / 16;    // padded floats per LDS row
  constexpr int NW = WG / 64;
  constexpr float Qb = QB<ABITS>::value;
  __shared__ float lds[NP > 1 ? R * ROWF : 1];
  __shared__ float redf[NW];
  __shared__ double redd[NW];
  // The absmean sum has slots of its own: without the transform no barrier separates it from
  // the sum of squares, whose slots slower waves of the row may still be reading.
  __shared__ double redd2[ABITS == 5 ? NW : 1];

  const int tid = threadIdx.x;
  const int rl = tid / T;
  const int t = tid % T;
  const int64_t ngroups = (M + R - 1) / R;
  float* rowlds = lds + rl * ROWF;

  float g[64];
  if constexpr (NM == 2) {
    // gamma in the thread's element order: 64 consecutive, or 8 chunks of 8 (no transform)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 q = *reinterpret_cast<const float4*>(
          gamma + (HT ? 64 * t + 4 * i : 8 * t + 8 * T * (i / 2) + 4 * (i % 2)));
      g[4 * i + 0] = q.x;
      g[4 * i + 1] = q.y;
      g[4 * i + 2] = q.z;
      g[4 * i + 3] = q.w;
    }
  }

  RowChunk<XT> cur, nxt;
  int64_t grp = blockIdx.x;
  auto load_group = [&](RowChunk<XT>& c, int64_t group) __attribute__((always_inline)) {
    const int64_t e0 = min(group * R + rl, M - 1) * K;
    if constexpr (HT) load_chunk<XT>(c, x, e0 + 64 * t);
    else load_chunk_strided<XT, T>(c, x, e0 + 8 * t);
  };
  if (grp < ngroups) load_group(cur, grp);
  for (; grp < ngroups; grp += gridDim.x) {
    const int64_t row = grp * R + rl;
    const bool valid = row < M;        // rows past M are computed from row M-1, never stored
    const int64_t ngrp = grp + gridDim.x;
    if (ngrp < ngroups) load_group(nxt, ngrp);

    float v[64];
    unpack_chunk<XT>(cur, v);
    float r = 1.0f;
    if constexpr (NM != 0) {
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < 64; ++j) ss = __builtin_fma((double)v[j], (double)v[j], ss);  // x^2 exact in fp64
      ss = row_sum<T>(ss, redd);
      r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
      if constexpr (NM == 2) {
#pragma unroll
        for (int j = 0; j < 64; ++j) v[j] *= g[j];
      }
    }

    // Phase 0: index bits 0..5 in registers.
    if constexpr (HT) stages<0, phase_desc(L, 0).a>(v);
    if constexpr (NP > 1) {
      lds_write<L, 0, ROWF>(v, rowlds, t);
      __syncthreads();
      lds_read<L, 1, ROWF>(v, rowlds, t);
      stages<Layout<L, 1>::c, Layout<L, 1>::a>(v);
    }
    if constexpr (NP > 2) {
      lds_write<L, 1, ROWF>(v, rowlds, t);
      __syncthreads();
      lds_read<L, 2, ROWF>(v, rowlds, t);
      stages<Layout<L, 2>::c, Layout<L, 2>::a>(v);
    }

    float amax = 0.0f;
    if constexpr (ABITS == 5) {
      double sa = 0.0;
#pragma unroll
      for (int j = 0; j < 64; ++j) sa += (double)fabsf(v[j]);
      amax = (float)(row_sum<T>(sa, redd2) / (double)K);  // the absmean statistic b
    } else {
#pragma unroll
      for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = row_max<T>(amax, redf);
    }

    const bool zero = amax < 0x1p-120f;     // also keeps Qb / amax finite
    // s = 0 quantises the whole row to 0
    const float s = zero ? 0.0f : (ABITS == 5 ? 1.0f / amax : Qb / amax);
    if (valid) {
      uint8_t* crow = codes + row * (int64_t)row_bytes<ABITS>(K);
      constexpr int LASTP = NP - 1;
      using LY = Layout<L, LASTP>;
      constexpr int RL = NP == 1 ? 64 : (1 << LY::c);  // run of consecutive elements in registers
      const int b = NP == 1 ? 64 * t : LY::base(t);
      if constexpr (!HT) {
#pragma unroll
        for (int i = 0; i < 8; ++i) store_run<ABITS, 8>(v + 8 * i, s, crow, 8 * (t + T * i));
      } else {
#pragma unroll
        for (int gi = 0; gi < 64 / RL; ++gi)
          store_run<ABITS, RL>(v + gi * RL, s, crow, NP == 1 ? b + gi * RL : b + LY::off(gi * RL));
      }
      if (t == 0)
        deq[row] = zero ? 0.0f : __fmul_rn(__fmul_rn(ABITS == 5 ? amax : amax / Qb, r), hK);
    }
    cur = nxt;
    // The next group reuses LDS and the reduction slots: every thread must be done with them.
    __syncthreads();
  }
}

template <int L, int ABITS, int XT, int NM>
__global__ __launch_bounds__(block_threads<L>()) void k_actquant_h(
    const void* __restrict__ x, int64_t M, const float* __restrict__ gamma, float eps, float hK,
    uint8_t* __restrict__ codes, float* __restrict__ deq) {
  actquant_rows<L, ABITS, XT, NM, true>(x, M, gamma, eps, hK, codes, deq);
}

template <int L, int ABITS, int XT, int NM>
__global__ __launch_bounds__(block_threads<L>()) void k_actquant_pow2(
    const void* __restrict__ x, int64_t M, const float* __restrict__ gamma, float eps,
    uint8_t* __restrict__ codes, float* __restrict__ deq) {
  actquant_rows<L, ABITS, XT, NM, false>(x, M, gamma, eps, 1.0f, codes, deq);
}

// Decode-regime H-BitLinear forward in one kernel (M <= R token rows, R = rows the block
// transforms at once: 1 for K = 16384, 2 for 8192, 4 for 4096).
// With a handful of rows, the two-kernel path pays the latency of a one-block activation
// kernel and then of the weight stream.  Here every block owns 16 output columns: it first
// issues the loads of its whole weight slice (16 rows x K/4 bytes, kept in registers), then
// transforms and quantises the M activation rows itself (the same code and the same fp32
// operations as k_actquant_h, so codes and deq are bit-identical), leaving the codes as
// int8 in LDS, and finally multiplies them with the weights on v_mfma_i32_16x16x64_i8.
// Every block repeats the (cheap) activation work; block 0 also writes the packed codes and
// deq to the caller's workspace, as the two-kernel path does.  The int32 sums are exact, so
// y equals the two-kernel path bit for bit.

__device__ __forceinline__ v4i dec_b_operand(uint32_t w) {
  return v4i{(int)((w << 6) & 0xC0C0C0C0u), (int)((w << 4) & 0xC0C0C0C0u), (int)((w << 2) & 0xC0C0C0C0u),
             (int)(w & 0xC0C0C0C0u)};
}

template <int L, int ABITS, int XT, int NM>
__global__ __launch_bounds__(block_threads<L>()) void k_decode_h(
    const void* __restrict__ x, int M, const float* __restrict__ gamma, float eps, float hK,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int N, uint8_t* __restrict__ codes,
    float* __restrict__ deq, float* __restrict__ y) {
  constexpr int K = 1 << L;
  constexpr int T = K / 64;           // threads per row
  constexpr int WG = block_threads<L>();
  constexpr int R = WG / T;           // rows transformed at once
  constexpr int NP = nphases(L);
  constexpr int ROWF = K + K / 16;
  constexpr int NW = WG / 64;
  constexpr int MMAX = DEC_MAX_GROUPS * R;
  constexpr int CST = K + 16;         // LDS stride of one row of int8 codes
  constexpr int G = K / (NW * 256);   // 256-deep weight groups per wave
  constexpr float Qb = QB<ABITS>::value;
  static_assert(NP == 3 && G >= 1, "the fused decode kernel covers K = 2^12 .. 2^15");
  // bf16 rows with unit gamma take the matrix-core transform of the activation kernel for such
  // rows (actquant_mfma.h), so that codes and deq are the ones that kernel writes
  constexpr bool HM = XT == 1 && NM != 2 && L <= 14;
  constexpr int LDSF = HM && HM_LDS_FLOATS > R * ROWF ? HM_LDS_FLOATS : R * ROWF;
  __shared__ __attribute__((aligned(16))) float lds[LDSF];
  __shared__ __attribute__((aligned(16))) int8_t cl[MMAX * CST];
  __shared__ float dl[MMAX];
  __shared__ float redf[NW];
  __shared__ double redd[NW];
  __shared__ double redd2[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = tid / T, t = tid % T;
  const int gq = lane >> 4, rq = lane & 15;   // MFMA lane coordinates
  const int n0 = blockIdx.x * 16;
  const uint8_t* brow = Wq + (int64_t)min(n0 + rq, N - 1) * (K / 4) + 16 * gq;
  uint4 wb[G];

  if constexpr (HM) {
    static_assert(HM_SLAB / K == R, "one slab holds the rows of one group");
    // 1) The slab of rows, then the block's weights (loads complete in issue order).
    uint4 raw[8];
    hm_load<L>(raw, static_cast<const uint16_t*>(x), M, 0, wave, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order
#pragma unroll
    for (int u = 0; u < G; ++u) wb[u] = *reinterpret_cast<const uint4*>(brow + 64 * (wave * G + u));
    // 2) Transform and quantise; int8 codes to LDS, and from block 0 the packed codes and deq.
    using P = HmPost<L>;
    constexpr int RL = P::RL;
    float v[64];
    HmStats st;
    hm_transform<L, ABITS, NM>(raw, hm_hadamard_b(lane, 0), hm_hadamard_b(lane, 1), lds, redf, redd, redd2, wave,
                               lane, v, st, [] {});
    const int E0 = P::thread_E(wave, lane);
    const int row = E0 >> L;
    // RMS factor 1/sqrt(mean(x^2) + eps): the mean in fp64, the reciprocal square root by
    // v_rsq_f32 (about one ulp; the sum of squares is already an fp32 sum per lane)
    const float r = NM != 0 ? __builtin_amdgcn_rsqf((float)(st.ss / (double)K + (double)eps)) : 1.0f;
    const bool zero = st.amax < 0x1p-120f;
    const float s = zero ? 0.0f : Qb / st.amax;
    if (row < M) {
      int8_t* crow = cl + row * CST;
#pragma unroll
      for (int gi = 0; gi < 64 / RL; ++gi) {
        const int k0 = (E0 + P::reg_E(gi * RL)) & (K - 1);
#pragma unroll
        for (int d = 0; d < RL / 4; ++d) {
          const float* q = v + gi * RL + 4 * d;
          const uint32_t q0 = rne_bits(q[0] * s, 12582912.0f), q1 = rne_bits(q[1] * s, 12582912.0f);
          const uint32_t q2 = rne_bits(q[2] * s, 12582912.0f), q3 = rne_bits(q[3] * s, 12582912.0f);
          const uint32_t lo = __builtin_amdgcn_perm(q1, q0, 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm(q3, q2, 0x04000c0cu);
          *reinterpret_cast<uint32_t*>(crow + k0 + 4 * d) = lo | hi;
        }
      }
      const float dq = zero ? 0.0f : __fmul_rn(__fmul_rn(st.amax / Qb, r), hK);
      const bool first = (E0 & (K - 1)) == 0;
      if (first) dl[row] = dq;
      if (blockIdx.x == 0) {
        uint8_t* grow = codes + (int64_t)row * row_bytes<ABITS>(K);
#pragma unroll
        for (int gi = 0; gi < 64 / RL; ++gi)
          store_run<ABITS, RL>(v + gi * RL, s, grow, (E0 + P::reg_E(gi * RL)) & (K - 1));
        if (first) deq[row] = dq;
      }
    }
    __syncthreads();  // codes and deq in LDS before the product
  } else {
  // 1) The first activation rows, then the block's weights (lane (gq, rq) of wave w holds
  //    chunk 4 (w G + u) + gq of row n0 + rq).  Loads complete in issue order, so the rows
  //    go first: the transform can start while the weights are still streaming in.
  RowChunk<XT> cur;
  load_chunk<XT>(cur, x, (int64_t)min(rl, M - 1) * K + 64 * t);
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order
#pragma unroll
  for (int u = 0; u < G; ++u) wb[u] = *reinterpret_cast<const uint4*>(brow + 64 * (wave * G + u));

  // 2) Activation rows, R at a time, exactly as k_actquant_h.
  float g[64];
  if constexpr (NM == 2) {
    const float4* gp = reinterpret_cast<const float4*>(gamma + 64 * t);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 q = gp[i];
      g[4 * i + 0] = q.x;
      g[4 * i + 1] = q.y;
      g[4 * i + 2] = q.z;
      g[4 * i + 3] = q.w;
    }
  }
  float* rowlds = lds + rl * ROWF;
  auto process_group = [&](int grp) {
    const int row = grp * R + rl;
    const bool valid = row < M;
    float v[64];
    unpack_chunk<XT>(cur, v);
    float r = 1.0f;
    if constexpr (NM != 0) {
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < 64; ++j) ss = __builtin_fma((double)v[j], (double)v[j], ss);
      ss = row_sum<T>(ss, redd);
      r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
      if constexpr (NM == 2) {
#pragma unroll
        for (int j = 0; j < 64; ++j) v[j] *= g[j];
      }
    }
    stages<0, phase_desc(L, 0).a>(v);
    lds_write<L, 0, ROWF>(v, rowlds, t);
    __syncthreads();
    lds_read<L, 1, ROWF>(v, rowlds, t);
    stages<Layout<L, 1>::c, Layout<L, 1>::a>(v);
    lds_write<L, 1, ROWF>(v, rowlds, t);
    __syncthreads();
    lds_read<L, 2, ROWF>(v, rowlds, t);
    stages<Layout<L, 2>::c, Layout<L, 2>::a>(v);

    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = row_max<T>(amax, redf);
    const bool zero = amax < 0x1p-120f;
    const float s = zero ? 0.0f : Qb / amax;
    using LY = Layout<L, 2>;
    constexpr int RL = 1 << LY::c;     // runs of consecutive elements in registers
    const int b = LY::base(t);
    if (valid) {
      // int8 codes (the low byte of the magic-number rounding, as in the INT8 packer)
      int8_t* crow = cl + row * CST;
#pragma unroll
      for (int gi = 0; gi < 64 / RL; ++gi) {
#pragma unroll
        for (int d = 0; d < RL / 4; ++d) {
          const float* q = v + gi * RL + 4 * d;
          const uint32_t q0 = rne_bits(q[0] * s, 12582912.0f), q1 = rne_bits(q[1] * s, 12582912.0f);
          const uint32_t q2 = rne_bits(q[2] * s, 12582912.0f), q3 = rne_bits(q[3] * s, 12582912.0f);
          const uint32_t lo = __builtin_amdgcn_perm(q1, q0, 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm(q3, q2, 0x04000c0cu);
          *reinterpret_cast<uint32_t*>(crow + b + LY::off(gi * RL) + 4 * d) = lo | hi;
        }
      }
      const float dq = zero ? 0.0f : __fmul_rn(__fmul_rn(amax / Qb, r), hK);
      if (t == 0) dl[row] = dq;
      if (blockIdx.x == 0) {
        uint8_t* grow = codes + (int64_t)row * row_bytes<ABITS>(K);
#pragma unroll
        for (int gi = 0; gi < 64 / RL; ++gi) store_run<ABITS, RL>(v + gi * RL, s, grow, b + LY::off(gi * RL));
        if (t == 0) deq[row] = dq;
      }
    }
    __syncthreads();  // LDS and reduction slots are reused by the next group
    };
  // Group 0 is peeled out of the loop so that the wait for its input, issued before the
  // weights, does not also wait for the weights.
  process_group(0);
  const int ngroups = (M + R - 1) / R;
  for (int grp = 1; grp < ngroups; ++grp) {
    load_chunk<XT>(cur, x, (int64_t)min(grp * R + rl, M - 1) * K + 64 * t);
    process_group(grp);
  }
  }

  // 3) The product: wave w covers groups [w G, w G + G) of K; step t of group C pairs k-block
  //    4 (4C + gq) + t of the codes with word t of the weight chunk 4C + gq.
  v4i acc4[4] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};  // independent chains
  const bool arow_ok = rq < M;
  const int8_t* arow = cl + rq * CST;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int C = wave * G + u;
    const uint32_t w4[4] = {wb[u].x, wb[u].y, wb[u].z, wb[u].w};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      v4i a = v4i{0, 0, 0, 0};
      if (arow_ok) {
        const uint4 av = *reinterpret_cast<const uint4*>(arow + 16 * (4 * (4 * C + gq) + tt));
        a = v4i{(int)av.x, (int)av.y, (int)av.z, (int)av.w};
      }
      acc4[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, dec_b_operand(w4[tt]), acc4[tt], 0, 0, 0);
    }
  }
  const v4i acc = acc4[0] + acc4[1] + acc4[2] + acc4[3];  // exact int32 sums

  // 4) Sum the waves' tiles (lane l, register v: token 4 (l / 16) + v, column l % 16) and
  //    dequantise: codes are int8 q and weights 64 t, so the sum is 64 times the product.
  int* red = reinterpret_cast<int*>(lds);
#pragma unroll
  for (int vv = 0; vv < 4; ++vv) red[(wave * 4 + vv) * 64 + lane] = acc[vv];
  __syncthreads();
  if (tid < 4 * 64) {
    const int vv = tid >> 6, l = tid & 63;
    int sum = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += red[(w * 4 + vv) * 64 + l];
    const int m = 4 * (l >> 4) + vv, n = n0 + (l & 15);
    if (m < M && n < N) y[(int64_t)m * N + n] = __fmul_rn(__fmul_rn((float)(sum >> 6), dl[m]), w_scale[0]);
  }
}

template <int L, int ABITS, int XT>
hipError_t launch_decode_l(const void* x, int64_t M, const float* gamma, float eps, int norm, const uint8_t* Wq,
                           const float* w_scale, int64_t N, uint8_t* codes, float* deq, float* y, hipStream_t s) {
  const float hK = (float)(1.0 / std::sqrt((double)(1 << L)));
  const dim3 grid((unsigned)((N + 15) / 16)), block(block_threads<L>());
  if (!norm)
    hipLaunchKernelGGL((k_decode_h<L, ABITS, XT, 0>), grid, block, 0, s, x, (int)M, gamma, eps, hK, Wq, w_scale,
                       (int)N, codes, deq, y);
  else if (gamma == nullptr)
    hipLaunchKernelGGL((k_decode_h<L, ABITS, XT, 1>), grid, block, 0, s, x, (int)M, gamma, eps, hK, Wq, w_scale,
                       (int)N, codes, deq, y);
  else
    hipLaunchKernelGGL((k_decode_h<L, ABITS, XT, 2>), grid, block, 0, s, x, (int)M, gamma, eps, hK, Wq, w_scale,
                       (int)N, codes, deq, y);
  return hipGetLastError();
}

template <int ABITS, int XT>
hipError_t dispatch_decode(int L, const void* x, int64_t M, const float* gamma, float eps, int norm,
                           const uint8_t* Wq, const float* w_scale, int64_t N, uint8_t* codes, float* deq, float* y,
                           hipStream_t s) {
  switch (L) {
    case 12: return launch_decode_l<12, ABITS, XT>(x, M, gamma, eps, norm, Wq, w_scale, N, codes, deq, y, s);
    case 13: return launch_decode_l<13, ABITS, XT>(x, M, gamma, eps, norm, Wq, w_scale, N, codes, deq, y, s);
    case 14: return launch_decode_l<14, ABITS, XT>(x, M, gamma, eps, norm, Wq, w_scale, N, codes, deq, y, s);
    default: return hipErrorInvalidValue;
  }
}

// BitLinear path (no transform), any K with K % 64 == 0: one 256-thread block per row,
// the row held in registers as NCH chunks of 8 consecutive elements per thread
// (K <= 2048 * NCH), or streamed twice from memory when NCH == 0.
template <int ABITS, int XT, int NCH>
__global__ __launch_bounds__(256) void k_actquant_plain(const void* __restrict__ x, int64_t M, int64_t K,
                                                        const float* __restrict__ gamma, float eps, int norm,
                                                        uint8_t* __restrict__ codes, float* __restrict__ deq) {
  constexpr int NCHR = NCH > 0 ? NCH : 1;
  __shared__ float redf[4];
  __shared__ double redd[4];
  __shared__ double redd2[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = (int)(K / 8);
  auto load8 = [&](int ch, float* o) {
    if constexpr (XT == 1) {
      uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + row * K + 8 * ch);
      o[0] = bf16lo(w.x); o[1] = bf16hi(w.x); o[2] = bf16lo(w.y); o[3] = bf16hi(w.y);
      o[4] = bf16lo(w.z); o[5] = bf16hi(w.z); o[6] = bf16lo(w.w); o[7] = bf16hi(w.w);
    } else {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + row * K + 8 * ch);
      float4 a = p[0], b = p[1];
      o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
  };
  auto scale8 = [&](int ch, float* o) {
    if (norm && gamma != nullptr) {
      const float4* gp = reinterpret_cast<const float4*>(gamma + 8 * ch);
      float4 a = gp[0], b = gp[1];
      o[0] *= a.x; o[1] *= a.y; o[2] *= a.z; o[3] *= a.w; o[4] *= b.x; o[5] *= b.y; o[6] *= b.z; o[7] *= b.w;
    }
  };
  float v[NCHR][8];
  double ss = 0.0, sa = 0.0;  // sa: sum |u| for the absmean statistic (ABITS 5)
  float amax = 0.0f;
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + 256 * c;
      if (ch < nch) {
        load8(ch, v[c]);
        if (norm) {
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = __builtin_fma((double)v[c][e], (double)v[c][e], ss);
        }
        scale8(ch, v[c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (ABITS == 5) sa += (double)fabsf(v[c][e]);
          else amax = fmaxf(amax, fabsf(v[c][e]));
        }
      }
    }
  } else {
    for (int ch = tid; ch < nch; ch += 256) {
      float o[8];
      load8(ch, o);
      if (norm) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fma((double)o[e], (double)o[e], ss);
      }
      scale8(ch, o);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (ABITS == 5) sa += (double)fabsf(o[e]);
        else amax = fmaxf(amax, fabsf(o[e]));
      }
    }
  }
  float r = 1.0f;
  if (norm) {
    ss = row_sum<256>(ss, redd);
    r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
  }
  if constexpr (ABITS == 5) amax = (float)(row_sum<256>(sa, redd2) / (double)K);  // the absmean b
  else amax = row_max<256>(amax, redf);
  constexpr float Qb = QB<ABITS>::value;
  const bool zero = amax < 0x1p-120f;
  const float s = zero ? 0.0f : (ABITS == 5 ? 1.0f / amax : Qb / amax);
  uint8_t* crow = codes + row * (int64_t)row_bytes<ABITS>((int)K);
  auto put = [&](int ch, const float* o) {
    if constexpr (ABITS == 6) {
      store_run<6, 8>(o, s, crow, 8 * ch);
    } else if constexpr (ABITS == 4 || ABITS == 5) {
      auto q = [&](float z) {  // absmean codes can exceed the INT4 range
        return ABITS == 5 ? rne_int(fminf(fmaxf(z * s, -8.0f), 7.0f)) : rne_int(z * s);
      };
      *reinterpret_cast<uint32_t*>(crow + 4 * ch) =
          pack8_a4(q(o[0]), q(o[1]), q(o[2]), q(o[3]), q(o[4]), q(o[5]), q(o[6]), q(o[7]));
    } else {
      *reinterpret_cast<uint2*>(crow + 8 * ch) =
          make_uint2(pack4_a8(rne_int(o[0] * s), rne_int(o[1] * s), rne_int(o[2] * s), rne_int(o[3] * s)),
                     pack4_a8(rne_int(o[4] * s), rne_int(o[5] * s), rne_int(o[6] * s), rne_int(o[7] * s)));
    }
  };
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + 256 * c;
      if (ch < nch) put(ch, v[c]);
    }
  } else {
    for (int ch = tid; ch < nch; ch += 256) {
      float o[8];
      load8(ch, o);
      scale8(ch, o);
      put(ch, o);
    }
  }
  if (tid == 0) deq[row] = zero ? 0.0f : __fmul_rn(ABITS == 5 ? amax : amax / Qb, r);
}

template <int L, int ABITS, int XT>
hipError_t launch_h(const void* x, int64_t M, const float* gamma, float eps, int norm, uint8_t* codes, float* deq,
                    hipStream_t s) {
  constexpr int K = 1 << L;
  constexpr int T = K / 64;
  constexpr int WG = block_threads<L>();
  constexpr int R = WG / T;
  const float hK = (float)(1.0 / std::sqrt((double)K));
  const int64_t groups = (M + R - 1) / R;
  // Persistent blocks, exactly as many as are resident at once: every block holds about
  // 68 KB of LDS (one 2^14-float row, or several shorter ones), so two fit in a CU's 160 KB
  // (one for K = 2^15), and each then walks its share of the row groups with the next
  // group's input prefetched.  Four times as many blocks, a few rounds of block launches,
  // measured 5-6 % slower at K = 2^14.
  const int64_t cap = L <= 14 ? 2 * CUS : CUS;
  const int64_t blocks = groups < cap ? groups : cap;
  const dim3 grid((unsigned)blocks), block(WG);
  if (!norm)
    hipLaunchKernelGGL((k_actquant_h<L, ABITS, XT, 0>), grid, block, 0, s, x, M, gamma, eps, hK, codes, deq);
  else if (gamma == nullptr)
    hipLaunchKernelGGL((k_actquant_h<L, ABITS, XT, 1>), grid, block, 0, s, x, M, gamma, eps, hK, codes, deq);
  else
    hipLaunchKernelGGL((k_actquant_h<L, ABITS, XT, 2>), grid, block, 0, s, x, M, gamma, eps, hK, codes, deq);
  return hipGetLastError();
}

template <int ABITS, int XT>
hipError_t dispatch_h(int L, const void* x, int64_t M, const float* gamma, float eps, int norm, uint8_t* codes,
                      float* deq, hipStream_t s) {
  switch (L) {
    case 6: return launch_h<6, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 7: return launch_h<7, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 8: return launch_h<8, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 9: return launch_h<9, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 10: return launch_h<10, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 11: return launch_h<11, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 12: return launch_h<12, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 13: return launch_h<13, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 14: return launch_h<14, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 15: return launch_h<15, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    default: return hipErrorInvalidValue;
  }
}

// BitLinear path for K = 2^L, 2^11 <= K <= 2^14: the persistent row kernel without the
// transform (64 consecutive elements per thread, reductions in registers and shuffles).
template <int L, int ABITS, int XT>
hipError_t launch_pow2(const void* x, int64_t M, const float* gamma, float eps, int norm, uint8_t* codes,
                       float* deq, hipStream_t s) {
  constexpr int K = 1 << L;
  constexpr int R = block_threads<L>() / (K / 64);
  const int64_t groups = (M + R - 1) / R;
  const int64_t blocks = groups < 2048 ? groups : 2048;
  const dim3 grid((unsigned)blocks), block(block_threads<L>());
  if (!norm)
    hipLaunchKernelGGL((k_actquant_pow2<L, ABITS, XT, 0>), grid, block, 0, s, x, M, gamma, eps, codes, deq);
  else if (gamma == nullptr)
    hipLaunchKernelGGL((k_actquant_pow2<L, ABITS, XT, 1>), grid, block, 0, s, x, M, gamma, eps, codes, deq);
  else
    hipLaunchKernelGGL((k_actquant_pow2<L, ABITS, XT, 2>), grid, block, 0, s, x, M, gamma, eps, codes, deq);
  return hipGetLastError();
}

template <int ABITS, int XT>
hipError_t dispatch_pow2(int L, const void* x, int64_t M, const float* gamma, float eps, int norm, uint8_t* codes,
                         float* deq, hipStream_t s) {
  switch (L) {
    case 11: return launch_pow2<11, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 12: return launch_pow2<12, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 13: return launch_pow2<13, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    case 14: return launch_pow2<14, ABITS, XT>(x, M, gamma, eps, norm, codes, deq, s);
    default: return hipErrorInvalidValue;
  }
}

template <int ABITS, int XT>
hipError_t dispatch_plain(const void* x, int64_t M, int64_t K, const float* gamma, float eps, int norm,
                          uint8_t* codes, float* deq, hipStream_t s) {
  const int64_t nch = K / 8;
  const dim3 grid((unsigned)M), block(256);
  if (nch <= 256)
    hipLaunchKernelGGL((k_actquant_plain<ABITS, XT, 1>), grid, block, 0, s, x, M, K, gamma, eps, norm, codes, deq);
  else if (nch <= 512)
    hipLaunchKernelGGL((k_actquant_plain<ABITS, XT, 2>), grid, block, 0, s, x, M, K, gamma, eps, norm, codes, deq);
  else if (nch <= 1024)
    hipLaunchKernelGGL((k_actquant_plain<ABITS, XT, 4>), grid, block, 0, s, x, M, K, gamma, eps, norm, codes, deq);
  else if (nch <= 2048)
    hipLaunchKernelGGL((k_actquant_plain<ABITS, XT, 8>), grid, block, 0, s, x, M, K, gamma, eps, norm, codes, deq);
  else
    hipLaunchKernelGGL((k_actquant_plain<ABITS, XT, 0>), grid, block, 0, s, x, M, K, gamma, eps, norm, codes, deq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_fused(const void* x, int xt, int64_t M, int64_t K, int norm, const float* gamma, float eps,
                               int abits, const uint8_t* Wq, const float* w_scale, int64_t N, uint8_t* codes,
                               float* deq, float* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  int L = 0;
  while ((int64_t(1) << L) < K) ++L;
  if (abits == 4)
    return xt ? dispatch_decode<4, 1>(L, x, M, gamma, eps, norm, Wq, w_scale, N, codes, deq, y, s)
              : dispatch_decode<4, 0>(L, x, M, gamma, eps, norm, Wq, w_scale, N, codes, deq, y, s);
  return xt ? dispatch_decode<8, 1>(L, x, M, gamma, eps, norm, Wq, w_scale, N, codes, deq, y, s)
            : dispatch_decode<8, 0>(L, x, M, gamma, eps, norm, Wq, w_scale, N, codes, deq, y, s);
}

hipError_t launch_actquant(const void* x, int xt, int64_t M, int64_t K, int norm, const float* gamma, float eps,
                           int abits, int use_h, uint8_t* codes, float* deq, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (actquant_mfma_ok(xt, K, gamma, norm, use_h))
    return launch_actquant_mfma(x, M, K, norm, eps, abits, codes, deq, s);
  if (use_h) {
    int L = 0;
    while ((int64_t(1) << L) < K) ++L;
    if (abits == 4)
      return xt ? dispatch_h<4, 1>(L, x, M, gamma, eps, norm, codes, deq, s)
                : dispatch_h<4, 0>(L, x, M, gamma, eps, norm, codes, deq, s);
    if (abits == 6)
      return xt ? dispatch_h<6, 1>(L, x, M, gamma, eps, norm, codes, deq, s)
                : dispatch_h<6, 0>(L, x, M, gamma, eps, norm, codes, deq, s);
    if (abits == 5)
      return xt ? dispatch_h<5, 1>(L, x, M, gamma, eps, norm, codes, deq, s)
                : dispatch_h<5, 0>(L, x, M, gamma, eps, norm, codes, deq, s);
    return xt ? dispatch_h<8, 1>(L, x, M, gamma, eps, norm, codes, deq, s)
              : dispatch_h<8, 0>(L, x, M, gamma, eps, norm, codes, deq, s);
  }
  int L = 0;
  while ((int64_t(1) << L) < K) ++L;
  if ((int64_t(1) << L) == K && L >= 11 && L <= 14) {
    if (abits == 4)
      return xt ? dispatch_pow2<4, 1>(L, x, M, gamma, eps, norm, codes, deq, s)
                : dispatch_pow2<4, 0>(L, x, M, gamma, eps, norm, codes, deq, s);
    if (abits == 6)
      return xt ? dispatch_pow2<6, 1>(L, x, M, gamma, eps, norm, codes, deq, s)
                : dispatch_pow2<6, 0>(L, x, M, gamma, eps, norm, codes, deq, s);
    if (abits == 5)
      return xt ? dispatch_pow2<5, 1>(L, x, M, gamma, eps, norm, codes, deq, s)
                : dispatch_pow2<5, 0>(L, x, M, gamma, eps, norm, codes, deq, s);
    return xt ? dispatch_pow2<8, 1>(L, x, M, gamma, eps, norm, codes, deq, s)
              : dispatch_pow2<8, 0>(L, x, M, gamma, eps, norm, codes, deq, s);
  }
  if (abits == 4)
    return xt ? dispatch_plain<4, 1>(x, M, K, gamma, eps, norm, codes, deq, s)
              : dispatch_plain<4, 0>(x, M, K, gamma, eps, norm, codes, deq, s);
  if (abits == 6)
    return xt ? dispatch_plain<6, 1>(x, M, K, gamma, eps, norm, codes, deq, s)
              : dispatch_plain<6, 0>(x, M, K, gamma, eps, norm, codes, deq, s);
  if (abits == 5)
    return xt ? dispatch_plain<5, 1>(x, M, K, gamma, eps, norm, codes, deq, s)
              : dispatch_plain<5, 0>(x, M, K, gamma, eps, norm, codes, deq, s);
  return xt ? dispatch_plain<8, 1>(x, M, K, gamma, eps, norm, codes, deq, s)
            : dispatch_plain<8, 0>(x, M, K, gamma, eps, norm, codes, deq, s);
}

}  // namespace hbl
