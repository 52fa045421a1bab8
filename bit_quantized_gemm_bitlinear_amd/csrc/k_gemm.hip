// k_gemm.hip — ternary-weight x INT4/INT8-activation GEMM with int32 accumulation on the
// gfx950 int8 matrix cores, plus the dequantisation epilogue.
//
// BitNet v2 write-up, section H-BitLinear模塊: the quantised activations multiply the
// ternary weights and the result is rescaled by the activation and weight scales;
// bitnet.cpp article: with weights in {-1, 0, 1} the product needs only additions.  On
// MI355X the dense int8 MFMA path is faster than any add-only scheme, so the codes are
// widened to int8 in registers and fed to v_mfma_i32_16x16x64_i8.
//
// Operand widening (exact; see the packed formats in hbl.h):
//   INT4 codes: word w of 8 nibbles -> (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0 give int8
//               bytes equal to 16*q, in natural k order for the two words of a group.
//   ternary:    word w of 16 2-bit fields -> (w << 6-2j) & 0xC0C0C0C0, j = 0..3, gives int8
//               bytes equal to 64*t, in natural k order.
//   INT8 codes: used as loaded.
// The int32 sum is therefore 1024*acc (INT4) or 64*acc (INT8); |acc| <= 127*K keeps it
// below 2^31 for K <= 2^17 and the final arithmetic shift is exact.
//
// Tiling: a 256-thread block computes a BM x BN tile of y; its four waves each own a
// (BM/2) x (BN/2) sub-tile of 16x16 MFMA tiles.  K advances in stages of 128: the next
// stage's A/B bytes are loaded from HBM into registers while the current stage is
// multiplied out of LDS (double-buffered, one barrier per stage).  LDS rows are padded so
// the fragment reads of 16 lanes from 16 rows hit distinct banks.
#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

constexpr int BK = 128;

// Block-to-tile order.  Blocks are dispatched round-robin over the 8 XCDs (block b runs on
// XCD b % 8), and each XCD has its own L2.  The remap gives every XCD a contiguous chunk of
// tile ids, and tile ids advance over groups of GM tile-rows so that the blocks resident
// on one XCD at the same time share A rows and B columns in its L2.
__device__ __forceinline__ void tile_of_block(int bid, int nblk, int ntm, int ntn, int GM, int& tm, int& tn) {
  constexpr int NXCD = 8;
  int t = bid;
  const int per = nblk / NXCD;
  if (bid < per * NXCD) t = (bid % NXCD) * per + bid / NXCD;
  const int group = t / (GM * ntn);
  const int first = group * GM;
  const int gm = min(ntm - first, GM);
  const int r = t - group * GM * ntn;
  tm = first + r % gm;
  tn = r / gm;
}

// One block computes a BM x BN tile of y with NWAVE waves laid out WR x WC; each wave owns
// (BM/WR) x (BN/WC) as 16x16 MFMA tiles.
template <int ABITS, int BM, int BN, int WR, int WC, int MODE>
__global__ __launch_bounds__(64 * WR * WC) void k_gemm(const uint8_t* __restrict__ A, const float* __restrict__ deq,
                                                       const uint8_t* __restrict__ B,
                                                       const float* __restrict__ w_scale, int M, int N, int K,
                                                       int32_t* __restrict__ acc_out, float* __restrict__ y) {
  constexpr int NT = 64 * WR * WC;                  // threads per block
  constexpr int AB = BK * ABITS / 8;                // bytes of one A row per stage
  constexpr int AS = AB + (ABITS == 4 ? 8 : 16);    // padded LDS row stride of A
  constexpr int BB = BK / 4;                        // bytes of one B row per stage
  constexpr int BS = BB + 8;                        // padded LDS row stride of B
  constexpr int WM = BM / WR, WN = BN / WC;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int ACH = AB / 16;                      // 16-byte chunks per A row per stage
  constexpr int BCH = BB / 16;
  constexpr int ALD = BM * ACH / NT;                // 16-byte loads per thread per stage
  constexpr int BLD = BN * BCH / NT;
  constexpr int SHIFT = ABITS == 4 ? 10 : 6;
  static_assert(ALD >= 1 && BLD >= 1 && ALD * NT == BM * ACH && BLD * NT == BN * BCH, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * AS];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * BS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WC, wn = wave % WC;
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  int tm, tn;
  tile_of_block(blockIdx.x, gridDim.x, ntm, ntn, 4, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t arow = (int64_t)K * ABITS / 8;
  const int64_t brow = K / 4;
  const int KT = (K + BK - 1) / BK;
  const bool last_half = (K % BK) != 0;

  uint4 ra[ALD], rb[BLD];
  auto gload = [&](int kt, bool half) {
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int e = tid + NT * i, r = e / ACH, c = e % ACH;
      const int gm = m0 + r;
      const bool ok = gm < M && (!half || c < ACH / 2);
      ra[i] = ok ? *reinterpret_cast<const uint4*>(A + (int64_t)gm * arow + (int64_t)kt * AB + 16 * c)
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
      const int e = tid + NT * i, r = e / BCH, c = e % BCH;
      const int gn = n0 + r;
      const bool ok = gn < N && (!half || c < BCH / 2);
      rb[i] = ok ? *reinterpret_cast<const uint4*>(B + (int64_t)gn * brow + (int64_t)kt * BB + 16 * c)
                 : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int e = tid + NT * i, r = e / ACH, c = e % ACH;
      uint8_t* d = &sA[buf][r * AS + 16 * c];
      if constexpr (ABITS == 8) {
        *reinterpret_cast<uint4*>(d) = ra[i];
      } else {
        reinterpret_cast<uint2*>(d)[0] = make_uint2(ra[i].x, ra[i].y);
        reinterpret_cast<uint2*>(d)[1] = make_uint2(ra[i].z, ra[i].w);
      }
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
      const int e = tid + NT * i, r = e / BCH, c = e % BCH;
      uint8_t* d = &sB[buf][r * BS + 16 * c];
      reinterpret_cast<uint2*>(d)[0] = make_uint2(rb[i].x, rb[i].y);
      reinterpret_cast<uint2*>(d)[1] = make_uint2(rb[i].z, rb[i].w);
    }
  };

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  auto compute_step = [&](int buf, int ks) {
    v4i b[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WN + 16 * j + (lane & 15);
      const uint32_t w = *reinterpret_cast<const uint32_t*>(&sB[buf][r * BS + ks * 16 + 4 * (lane >> 4)]);
      b[j] = v4i{(int)((w << 6) & 0xC0C0C0C0u), (int)((w << 4) & 0xC0C0C0C0u), (int)((w << 2) & 0xC0C0C0C0u),
                 (int)(w & 0xC0C0C0C0u)};
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      v4i a;
      const int r = wm * WM + 16 * i + (lane & 15);
      if constexpr (ABITS == 4) {
        const uint2 w = *reinterpret_cast<const uint2*>(&sA[buf][r * AS + ks * 32 + 8 * (lane >> 4)]);
        a = v4i{(int)((w.x << 4) & 0xF0F0F0F0u), (int)(w.x & 0xF0F0F0F0u), (int)((w.y << 4) & 0xF0F0F0F0u),
                (int)(w.y & 0xF0F0F0F0u)};
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(&sA[buf][r * AS + ks * 64 + 16 * (lane >> 4)]);
        a = v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j], acc[i][j], 0, 0, 0);
    }
  };

  gload(0, KT == 1 && last_half);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool has_next = kt + 1 < KT;
    if (has_next) gload(kt + 1, kt + 1 == KT - 1 && last_half);
    const int buf = kt & 1;
    compute_step(buf, 0);
    if (!(kt == KT - 1 && last_half)) compute_step(buf, 1);
    if (has_next) swrite(buf ^ 1);
    __syncthreads();
  }

  float alpha = 0.0f;
  if constexpr (MODE == 1) alpha = w_scale[0];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + wm * WM + 16 * i + 4 * (lane >> 4) + v;
      if (m >= M) continue;
      float dm = 0.0f;
      if constexpr (MODE == 1) dm = deq[m];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + 16 * j + (lane & 15);
        if (n >= N) continue;
        const int val = acc[i][j][v] >> SHIFT;
        if constexpr (MODE == 0) {
          acc_out[(int64_t)m * N + n] = val;
        } else {
          y[(int64_t)m * N + n] = __fmul_rn(__fmul_rn((float)val, dm), alpha);
        }
      }
    }
  }
}

template <int ABITS, int BM, int BN, int WR, int WC, int MODE>
hipError_t launch_cfg(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale, int64_t M,
                      int64_t K, int64_t N, int32_t* acc, float* y, hipStream_t s) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm<ABITS, BM, BN, WR, WC, MODE>), dim3((unsigned)tiles), dim3(64 * WR * WC), 0, s, codes,
                     deq, Wq, w_scale, (int)M, (int)N, (int)K, acc, y);
  return hipGetLastError();
}

// Tile choice: a 256x256 tile multiplies at roughly twice the rate of a 128x128 tile, so it
// wins unless it leaves most of the 256 CUs idle.
inline bool use_big_tiles(int64_t M, int64_t N) {
  constexpr int64_t CUS = 256;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const double time256 = (double)((t256 + CUS - 1) / CUS) * 4.0 / 2.0;
  const double time128 = (double)((t128 + CUS - 1) / CUS) * 1.0;
  return time256 <= time128;
}

template <int ABITS, int MODE>
hipError_t launch(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale, int64_t M,
                  int64_t K, int64_t N, int32_t* acc, float* y, hipStream_t s) {
  if (use_big_tiles(M, N))
    return launch_cfg<ABITS, 256, 256, 2, 4, MODE>(codes, deq, Wq, w_scale, M, K, N, acc, y, s);
  return launch_cfg<ABITS, 128, 128, 2, 2, MODE>(codes, deq, Wq, w_scale, M, K, N, acc, y, s);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale, int64_t M,
                       int64_t K, int64_t N, int abits, int32_t* acc, float* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (acc != nullptr)
    return abits == 4 ? launch<4, 0>(codes, deq, Wq, w_scale, M, K, N, acc, y, s)
                      : launch<8, 0>(codes, deq, Wq, w_scale, M, K, N, acc, y, s);
  return abits == 4 ? launch<4, 1>(codes, deq, Wq, w_scale, M, K, N, acc, y, s)
                    : launch<8, 1>(codes, deq, Wq, w_scale, M, K, N, acc, y, s);
}

}  // namespace hbl
