// k_gemv.hip — the ternary GEMM in the decode regime (M <= 64 token rows).
//
// With few tokens the layer is bound by streaming the 2-bit weights from HBM, the case the
// bitnet.cpp article and the BitNet v2 write-up describe for low-bit inference (weights read
// once per generated token).  The kernel reads every weight byte exactly once, with 16-byte
// loads issued in batches so that many are in flight per CU, and still multiplies on the
// int8 matrix cores (v_mfma_i32_16x16x64_i8), whose rate keeps the arithmetic well below the
// load time up to M = 64.
//
// Block b owns 16 output columns (weight rows n0 .. n0+15) and all M tokens; its waves (8 for
// M <= 16, 16 above, where each lane also loads the codes of up to four token tiles) split K
// and their int32 tiles are summed in LDS.  The integer sum is exact, so the result
// equals the large-M kernel bit for bit.
//
// K order inside a 256-deep group C: lane (g, r) = (lane / 16, lane % 16) loads the 16-byte
// weight chunk 4C + g of row r (64 weights) and the matching 64 codes of token rows r,
// r + 16, ...; MFMA step t of the group multiplies the 16-deep block t of those chunks.  Both
// operands use the same assignment, so each step pairs codes and weights of the same k.
#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

template <int ABITS>
struct AChunk;  // one lane's 64 codes of a 64-deep chunk
template <>
struct AChunk<4> {
  uint4 v[2];
};
template <>
struct AChunk<8> {
  uint4 v[4];
};

// 16 codes of k-block t (0..3) widened to int8 MFMA operand bytes (16*q for INT4, q for INT8).
template <int ABITS>
__device__ __forceinline__ v4i a_operand(const AChunk<ABITS>& c, int t) {
  if constexpr (ABITS == 4) {
    const uint4 h = c.v[t >> 1];
    const uint32_t x = (t & 1) ? h.z : h.x, y = (t & 1) ? h.w : h.y;
    return v4i{(int)((x << 4) & 0xF0F0F0F0u), (int)(x & 0xF0F0F0F0u), (int)((y << 4) & 0xF0F0F0F0u),
               (int)(y & 0xF0F0F0F0u)};
  } else {
    const uint4 h = c.v[t];
    return v4i{(int)h.x, (int)h.y, (int)h.z, (int)h.w};
  }
}

// One 32-bit word of 16 packed weights -> int8 operand bytes 64*t in natural k order.
__device__ __forceinline__ v4i b_operand(uint32_t w) {
  return v4i{(int)((w << 6) & 0xC0C0C0C0u), (int)((w << 4) & 0xC0C0C0C0u), (int)((w << 2) & 0xC0C0C0C0u),
             (int)(w & 0xC0C0C0C0u)};
}

// MT: 16-row token tiles (M <= 16 MT); U: 256-deep groups loaded per batch; GV_WAVES waves.
template <int ABITS, int MT, int U, int GV_WAVES, int MODE>
__global__ __launch_bounds__(64 * GV_WAVES) void k_gemv(const uint8_t* __restrict__ A, const float* __restrict__ deq,
                                                        const uint8_t* __restrict__ B,
                                                        const float* __restrict__ w_scale, int M, int N, int K,
                                                        int32_t* __restrict__ acc_out, float* __restrict__ y) {
  constexpr int SHIFT = ABITS == 4 ? 10 : 6;
  constexpr int ACB = 64 * ABITS / 8;  // code bytes of one 64-deep chunk
  __shared__ int32_t red[GV_WAVES][MT * 4][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int nchunks = K / 64;
  const int ngroups = (nchunks + 3) / 4;
  const int per = (ngroups + GV_WAVES - 1) / GV_WAVES;
  const int c0 = wave * per, c1 = min(ngroups, c0 + per);

  // Weight rows past N are clamped to the last one; their sums are never stored.  Token rows
  // past M are not loaded at all (their codes are taken as zero), so a small M issues only the
  // code loads it needs.
  const uint8_t* brow = B + (int64_t)min(n0 + r, N - 1) * (K / 4) + 16 * g;
  const uint8_t* arow[MT];
  bool alive[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    alive[mt] = 16 * mt + r < M;
    arow[mt] = A + (int64_t)min(16 * mt + r, M - 1) * (K * ABITS / 8) + ACB * g;
  }

  v4i acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v4i{0, 0, 0, 0};

  for (int cb = c0; cb < c1; cb += U) {
    uint4 wb[U];
    AChunk<ABITS> ac[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int chunk = 4 * (cb + u) + g;
      const bool ok = cb + u < c1 && chunk < nchunks;
      wb[u] = ok ? *reinterpret_cast<const uint4*>(brow + (int64_t)64 * (cb + u)) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < ACB / 16; ++q)
          ac[u][mt].v[q] = ok && alive[mt] ? *reinterpret_cast<const uint4*>(arow[mt] + (int64_t)4 * ACB * (cb + u) + 16 * q)
                              : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w4[4] = {wb[u].x, wb[u].y, wb[u].z, wb[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4i b = b_operand(w4[t]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_operand<ABITS>(ac[u][mt], t), b, acc[mt], 0, 0, 0);
      }
    }
  }

  // Result layout: register v of lane l holds token 16 mt + 4 (l / 16) + v, column l % 16.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * mt + v][lane] = acc[mt][v];
  __syncthreads();
  const float alpha = MODE == 1 ? w_scale[0] : 0.0f;
  for (int e = threadIdx.x; e < MT * 4 * 64; e += 64 * GV_WAVES) {
    const int mv = e >> 6, l = e & 63;
    int s = 0;
#pragma unroll
    for (int w = 0; w < GV_WAVES; ++w) s += red[w][mv][l];
    const int m = 16 * (mv >> 2) + 4 * (l >> 4) + (mv & 3);
    const int n = n0 + (l & 15);
    if (m >= M || n >= N) continue;
    const int val = s >> SHIFT;
    if constexpr (MODE == 0) acc_out[(int64_t)m * N + n] = val;
    else y[(int64_t)m * N + n] = __fmul_rn(__fmul_rn((float)val, deq[m]), alpha);
  }
}

template <int ABITS, int MODE>
hipError_t launch_mode(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale, int64_t M,
                       int64_t K, int64_t N, int32_t* acc, float* y, hipStream_t s) {
  const dim3 grid((unsigned)((N + 15) / 16));
  const int mt = (int)((M + 15) / 16);
  if (mt == 1)
    hipLaunchKernelGGL((k_gemv<ABITS, 1, 4, 8, MODE>), grid, dim3(64 * 8), 0, s, codes, deq, Wq, w_scale, (int)M,
                       (int)N, (int)K, acc, y);
  else if (mt == 2)
    hipLaunchKernelGGL((k_gemv<ABITS, 2, 4, 16, MODE>), grid, dim3(64 * 16), 0, s, codes, deq, Wq, w_scale, (int)M,
                       (int)N, (int)K, acc, y);
  else
    hipLaunchKernelGGL((k_gemv<ABITS, 4, 2, 16, MODE>), grid, dim3(64 * 16), 0, s, codes, deq, Wq, w_scale, (int)M,
                       (int)N, (int)K, acc, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale, int64_t M,
                       int64_t K, int64_t N, int abits, int32_t* acc, float* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (acc != nullptr)
    return abits == 4 ? launch_mode<4, 0>(codes, deq, Wq, w_scale, M, K, N, acc, y, s)
                      : launch_mode<8, 0>(codes, deq, Wq, w_scale, M, K, N, acc, y, s);
  return abits == 4 ? launch_mode<4, 1>(codes, deq, Wq, w_scale, M, K, N, acc, y, s)
                    : launch_mode<8, 1>(codes, deq, Wq, w_scale, M, K, N, acc, y, s);
}

}  // namespace hbl
