// k_gemm.hip — ternary-weight x INT4/INT8-activation GEMM with int32 accumulation on the
// gfx950 int8 matrix cores, plus the dequantisation epilogue.
//
// BitNet v2 write-up, section H-BitLinear模塊: the quantised activations multiply the
// ternary weights and the result is rescaled by the activation and weight scales;
// bitnet.cpp article: with weights in {-1, 0, 1} the product needs only additions.  On
// MI355X the dense int8 MFMA path is faster than any add-only scheme, so the codes are
// widened to int8 in registers and fed to v_mfma_i32_32x32x32_i8.
//
// Operand widening (exact; see the packed formats in hbl.h):
//   INT4 codes: word w of 8 nibbles -> (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0 give int8
//               bytes equal to 16*q, in natural k order for the two words of a group.
//   ternary:    word w of 16 2-bit fields -> (w << 6-2j) & 0xC0C0C0C0, j = 0..3, gives int8
//               bytes equal to 64*t, in natural k order.
//   INT8 codes: used as loaded.
// The int32 sum is therefore 1024*acc (INT4) or 64*acc (INT8); |acc| <= 127*K keeps it
// below 2^31 for K <= 2^17 and the final arithmetic shift is exact.  Pairs of words are
// shifted as one 64-bit value (see fmma below).  When K is a multiple of the stage depth
// the kernel is instantiated without the K-tail masks on its loads.
//
// Tiling for large problems: a 512-thread block computes a 256 x 256 tile of y; its eight
// waves (2 x 4) each own a 128 x 64 sub-tile of 32x32 MFMA tiles (128 int32 accumulators
// per lane, two waves per SIMD).  The fused gate/up GEMM uses 128 x 256 tiles of four such
// waves, two blocks per CU (see launch).  On gfx950 every VALU instruction issued beside an MFMA
// costs issue time, so the 32x32x32 shape (twice the work per instruction of 16x16x64)
// and a wide wave tile (each decoded fragment feeds 2-4 MFMAs) keep the decode overhead
// low.  K advances in LDS stages (256 deep for INT4, 128 for INT8), double buffered with
// one barrier per stage.  Buffer loads fetch each stage two stages ahead into one of two
// register sets, and the stage loaded during the previous one is stored to LDS in pieces
// between the current stage's k-steps; each 32-deep step's fragments are read from LDS one
// step ahead.  LDS rows are padded so the fragment reads hit distinct banks.  Small
// problems use 128 x 128 tiles (4 waves) so that more CUs get work.
//
// Epilogues (MODE): 0 stores the int32 product, 1 the dequantised y.  2 and 3 are the fused
// gate/up projection of the FFN block: B holds the gate and up weights interleaved in blocks
// of 32 rows, so the two 32-column MFMA tiles of a wave hold g and u for the same outputs in
// the same lanes; the epilogue dequantises both with their own weight scales and stores
// h = silu(g) * u once (fp32 for 2, bf16 for 3) instead of writing g and u.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

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

// Operand fragments of one 32-deep k-step for one wave: per 32-row A tile the lane's 16
// codes (INT4: 8 packed bytes, INT8: 16 bytes) and per 32-column B tile the lane's 16 packed
// weights (one 32-bit word), straight from LDS.
template <int ABITS, int TM, int TN>
struct Frag {
  typename std::conditional<ABITS == 4, uint2, uint4>::type a[TM];
  uint32_t b[TN];
};

// One block computes a BM x BN tile of y with WR x WC waves; each wave owns
// (BM/WR) x (BN/WC) as 32x32 tiles of v_mfma_i32_32x32x32_i8 (lane l holds row/column l%32
// and the 16 k-values 16*(l/32) .. +15 of the 32-deep step; result row 8(v/4)+4(l/32)+v%4,
// column l%32 in accumulator register v).  K advances in stages of BK (BK/32 k-steps).
//
// SPLIT: the block multiplies only the stages [blockIdx.y * kt_per, + kt_per) of K and adds
// its int32 result into acc_out with atomics (exact: integer sums do not depend on order);
// the caller zeroes acc_out before and, for MODE 1, dequantises it after.
template <int ABITS, int BM, int BN, int WR, int WC, int BK, int MODE, bool FULLK, bool SPLIT>
__global__ __launch_bounds__(64 * WR * WC) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm(const uint8_t* __restrict__ A, const float* __restrict__ deq,
                                                       const uint8_t* __restrict__ B,
                                                       const float* __restrict__ w_scale,
                                                       const float* __restrict__ w_scale_up, int M, int N, int K,
                                                       int32_t* __restrict__ acc_out, void* __restrict__ out,
                                                       int kt_per) {
  constexpr int NT = 64 * WR * WC;                  // threads per block
  constexpr int KS = BK / 32;                       // k-steps per stage
  constexpr int AB = BK * ABITS / 8;                // bytes of one A row per stage
  constexpr int AS = AB + (ABITS == 4 ? 8 : 16);    // padded LDS row stride of A (b64 / b128 reads)
  constexpr int BB = BK / 4;                        // bytes of one B row per stage
  constexpr int BS = BB + 4;                        // odd dword stride: 32 lanes, 32 banks
  constexpr int WM = BM / WR, WN = BN / WC;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int ACH = AB / 16;                      // 16-byte chunks per A row per stage
  constexpr int BCH = BB / 16;
  constexpr int ALD = BM * ACH / NT;                // 16-byte loads per thread per stage
  constexpr int BLD = BN * BCH / NT;
  constexpr int SHIFT = ABITS == 4 ? 10 : 6;
  static_assert(KS % 2 == 0, "stages hold an even number of k-steps");
  static_assert(ALD >= 1 && BLD >= 1 && ALD * NT == BM * ACH && BLD * NT == BN * BCH, "tile/thread mismatch");
  static_assert(MODE < 2 || WN == 64, "the fused gate/up epilogue pairs a wave's two 32-column tiles");
  static_assert(!SPLIT || MODE < 2, "split K is for the int32 and dequant epilogues");

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
  const int last_k64 = (K - (KT - 1) * BK) / 64;   // 64-deep slices in the last stage
  const int kb = SPLIT ? (int)blockIdx.y * kt_per : 0;   // this block's first stage
  const int KTL = SPLIT ? min(KT - kb, kt_per) : KT;     // and its number of stages

  // Per-thread global sources, 32-bit offsets from the tile's first row.  Rows past M
  // (columns past N) are clamped to the last valid one: their products land in accumulator
  // rows (columns) the epilogue never stores.
  const uint8_t* Ablk = A + (int64_t)m0 * arow;
  const uint8_t* Bblk = B + (int64_t)n0 * brow;
  uint32_t aoff[ALD];
#pragma unroll
  for (int i = 0; i < ALD; ++i) {
    const int e = tid + NT * i, r = e / ACH, c = e % ACH;
    aoff[i] = (uint32_t)(min(r, M - 1 - m0) * arow + 16 * c);
  }
  uint32_t boff[BLD];
#pragma unroll
  for (int i = 0; i < BLD; ++i) {
    const int e = tid + NT * i, r = e / BCH, c = e % BCH;
    boff[i] = (uint32_t)(min(r, N - 1 - n0) * brow + 16 * c);
  }

  // Buffer resources over the tile's rows of A and B: the loads take the loop-invariant
  // per-lane offsets above and the stage offset as a scalar.
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Ablk), (short)0, (int)(min(BM, M - m0) * arow), 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Bblk), (short)0, (int)(min(BN, N - n0) * brow), 0x00020000);
  // Two register sets stage the global loads: set S receives stage kt + 2 while the other
  // set, loaded a stage earlier, is stored to LDS.  S is a compile-time constant at every
  // call; the sets are chosen with if constexpr and copied element by element, because a
  // run-time subscript or pointer select on them makes the compiler keep them in memory.
  struct Stage {
    uint4 a[ALD], b[BLD];
  };
  Stage st0, st1;
  auto stg = [&](auto S) __attribute__((always_inline)) -> Stage& {
    if constexpr (decltype(S)::value == 0) return st0;
    else return st1;
  };
  // Load stage kt.  In the last stage only its first n64 64-deep slices exist; the rest of
  // the stage is zero-filled (zero weights and codes contribute nothing).
  auto gload = [&](auto S, int kt, int n64) __attribute__((always_inline)) {
    Stage& r = stg(S);
    const int va = n64 * 64 * ABITS / 8 / 16, vb = n64;
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const v4u v = FULLK || (int)((tid + NT * i) % ACH) < va
                        ? __builtin_amdgcn_raw_buffer_load_b128(rA, aoff[i], kt * AB, 0)
                        : v4u{0, 0, 0, 0};
      r.a[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
      const v4u v = FULLK || (int)((tid + NT * i) % BCH) < vb
                        ? __builtin_amdgcn_raw_buffer_load_b128(rB, boff[i], kt * BB, 0)
                        : v4u{0, 0, 0, 0};
      r.b[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  // FULLK (K a multiple of BK): every stage is whole, and the loads carry no masks.
  auto load_stage = [&](auto S, int kt) __attribute__((always_inline)) {
    if constexpr (FULLK) gload(S, kt, BK / 64);
    else gload(S, kt, kt == KT - 1 ? last_k64 : BK / 64);
  };
  // Store chunks [c0, c1) of register set S (A chunks first, then B chunks) into LDS buffer buf.
  auto swrite = [&](auto S, int buf, int c0 = 0, int c1 = 1 << 20) __attribute__((always_inline)) {
    const Stage& r = stg(S);
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      if (i < c0 || i >= c1) continue;
      const int e = tid + NT * i;
      uint8_t* d = &sA[buf][(e / ACH) * AS + 16 * (e % ACH)];
      if constexpr (ABITS == 8) {
        *reinterpret_cast<uint4*>(d) = make_uint4(r.a[i].x, r.a[i].y, r.a[i].z, r.a[i].w);
      } else {
        reinterpret_cast<uint2*>(d)[0] = make_uint2(r.a[i].x, r.a[i].y);
        reinterpret_cast<uint2*>(d)[1] = make_uint2(r.a[i].z, r.a[i].w);
      }
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
      if (ALD + i < c0 || ALD + i >= c1) continue;
      const int e = tid + NT * i;
      uint32_t* d = reinterpret_cast<uint32_t*>(&sB[buf][(e / BCH) * BS + 16 * (e % BCH)]);
      d[0] = r.b[i].x;
      d[1] = r.b[i].y;
      d[2] = r.b[i].z;
      d[3] = r.b[i].w;
    }
  };

  using F = Frag<ABITS, TM, TN>;
  constexpr int AKS = ABITS == 4 ? 16 : 32;         // A bytes per row per 32-deep step
  const int arow0 = (wm * WM + (lane & 31)) * AS + (AKS / 2) * (lane >> 5);
  const int brow0 = (wn * WN + (lane & 31)) * BS + 4 * (lane >> 5);
  auto fread = [&](int buf, int ks, F& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint8_t* p = &sA[buf][arow0 + 32 * i * AS + ks * AKS];
      if constexpr (ABITS == 4) f.a[i] = *reinterpret_cast<const uint2*>(p);
      else f.a[i] = *reinterpret_cast<const uint4*>(p);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const uint32_t*>(&sB[buf][brow0 + 32 * j * BS + ks * 8]);
  };

  // The accumulators live in the AGPR file: the empty asm with an "a" constraint makes the
  // compiler select the AGPR form of the MFMAs, so the matrix core reads and writes them
  // outside the VGPRs the widening and address arithmetic use (about 3 % faster than VGPR
  // accumulators at the same occupancy; 128 AGPRs + at most 128 VGPRs per lane).
  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = v16i{};
      asm volatile("" : "+a"(acc[i][j]));
    }

  // Widening with 64-bit shifts: one v_lshlrev_b64 shifts two words, and the byte masks clear
  // the bits that cross from the low word into the high one (they land below the kept bits
  // of the high word's first byte).  The two words of an INT4 fragment share a shift, and so
  // do the weight words of tiles 2p and 2p+1.  The empty asm keeps the compiler from
  // splitting each shift back into two 32-bit ones (it sees that the crossing bits are
  // masked off); this saves 7 of 38 widening instructions per 32-deep step of a wave.
  auto fmma = [&](const F& f) {
    v4i b[TN];
#pragma unroll
    for (int j = 0; j < TN; j += 2) {
      if (j + 1 < TN) {
        const uint64_t w = (uint64_t)f.b[j] | ((uint64_t)f.b[j + 1] << 32);
        uint64_t w6 = w << 6, w4 = w << 4, w2 = w << 2;
        asm volatile("" : "+v"(w6), "+v"(w4), "+v"(w2));  // keep each shift one 64-bit op
        b[j] = v4i{(int)((uint32_t)w6 & 0xC0C0C0C0u), (int)((uint32_t)w4 & 0xC0C0C0C0u),
                   (int)((uint32_t)w2 & 0xC0C0C0C0u), (int)((uint32_t)w & 0xC0C0C0C0u)};
        b[j + 1] = v4i{(int)((uint32_t)(w6 >> 32) & 0xC0C0C0C0u), (int)((uint32_t)(w4 >> 32) & 0xC0C0C0C0u),
                       (int)((uint32_t)(w2 >> 32) & 0xC0C0C0C0u), (int)((uint32_t)(w >> 32) & 0xC0C0C0C0u)};
      } else {
        const uint32_t w = f.b[j];
        b[j] = v4i{(int)((w << 6) & 0xC0C0C0C0u), (int)((w << 4) & 0xC0C0C0C0u), (int)((w << 2) & 0xC0C0C0C0u),
                   (int)(w & 0xC0C0C0C0u)};
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      v4i a;
      if constexpr (ABITS == 4) {
        const uint64_t w = (uint64_t)f.a[i].x | ((uint64_t)f.a[i].y << 32);
        uint64_t w4 = w << 4;
        asm volatile("" : "+v"(w4));
        a = v4i{(int)((uint32_t)w4 & 0xF0F0F0F0u), (int)((uint32_t)w & 0xF0F0F0F0u),
                (int)((uint32_t)(w4 >> 32) & 0xF0F0F0F0u), (int)((uint32_t)(w >> 32) & 0xF0F0F0F0u)};
      } else {
        const uint4 w = f.a[i];
        a = v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[j], acc[i][j], 0, 0, 0);
    }
  };

  // Software pipeline over two LDS buffers and two register sets: the loads of stage kt + 2
  // are issued at the start of stage kt, and stage kt + 1 (loaded during stage kt - 1) is
  // stored into the other LDS buffer a few chunks after each pair of k-steps of kt, so a
  // load has about a stage to arrive and the LDS stores are spread between the MFMAs.
  // Within a stage the k-steps ping-pong between two fragment sets, each read from LDS one
  // step ahead.  Loads and stores are unconditional (past the last stage they reload it and
  // store into the idle buffer), so the compiler's memory-counter waits stay exact: a
  // branch around them would make it wait for the loads just issued as well.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  F f0, f1;
  auto stage = [&](auto S, int kt) __attribute__((always_inline)) {  // kt counts this block's stages
    constexpr int set = decltype(S)::value;
    const int buf = kt & 1;
    load_stage(S, kb + min(kt + 2, KTL - 1));
    constexpr int NCH = ALD + BLD, PER = (NCH + KS / 2 - 1) / (KS / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      fread(buf, ks + 1, f1);
      fmma(f0);
      if (ks + 2 < KS) fread(buf, ks + 2, f0);
      swrite(std::integral_constant<int, 1 - set>{}, buf ^ 1, (ks / 2) * PER, (ks / 2 + 1) * PER);
      fmma(f1);
    }
    __syncthreads();
    fread(buf ^ 1, 0, f0);
  };
  load_stage(I0{}, kb);
  load_stage(I1{}, kb + min(1, KTL - 1));
  swrite(I0{}, 0);
  __syncthreads();
  fread(0, 0, f0);
  int kt = 0;
  for (; kt + 1 < KTL; kt += 2) {
    stage(I0{}, kt);
    stage(I1{}, kt + 1);
  }
  if (kt < KTL) stage(I0{}, kt);

  // The epilogue takes the lane index afresh (v_mbcnt) rather than keeping the main loop's
  // lane-derived values live across it, which at 128 VGPRs made the compiler spill them.
  const int el = __lane_id();
  if constexpr (MODE >= 2) {
    // Fused gate/up: B rows n0 + 64*wn + [0, 32) are gate rows and [32, 64) the up rows of
    // the same 32 outputs h[:, n0/2 + 32*wn + (lane % 32)]; N here counts both (2F rows).
    const float ag = w_scale[0], au = w_scale_up[0];
    const int F = N / 2;
    const int n = n0 / 2 + wn * 32 + (el & 31);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * (el >> 5) + (v & 3);
        if (m >= M || n >= F) continue;
        const float dm = deq[m];
        const float g = __fmul_rn(__fmul_rn((float)(acc[i][0][v] >> SHIFT), dm), ag);
        const float u = __fmul_rn(__fmul_rn((float)(acc[i][1][v] >> SHIFT), dm), au);
        const float h = silu_mul(g, u);
        if constexpr (MODE == 2) static_cast<float*>(out)[(int64_t)m * F + n] = h;
        else static_cast<uint16_t*>(out)[(int64_t)m * F + n] = f32_to_bf16_rne(h);
      }
    }
    return;
  }
  float alpha = 0.0f;
  if constexpr (MODE == 1) alpha = w_scale[0];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * (el >> 5) + (v & 3);
      if (m >= M) continue;
      float dm = 0.0f;
      if constexpr (MODE == 1) dm = deq[m];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + 32 * j + (el & 31);
        if (n >= N) continue;
        const int val = acc[i][j][v] >> SHIFT;
        if constexpr (SPLIT) {
          atomicAdd(&acc_out[(int64_t)m * N + n], val);
        } else if constexpr (MODE == 0) {
          acc_out[(int64_t)m * N + n] = val;
        } else {
          static_cast<float*>(out)[(int64_t)m * N + n] = __fmul_rn(__fmul_rn((float)val, dm), alpha);
        }
      }
    }
  }
}

template <int ABITS, int BM, int BN, int WR, int WC, int BK, int MODE>
hipError_t launch_cfg(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale,
                      const float* w_scale_up, int64_t M, int64_t K, int64_t N, int32_t* acc, void* out,
                      int splits, hipStream_t s) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int KT = (int)((K + BK - 1) / BK);
  if constexpr (MODE <= 1) {
    if (splits > 1) {
      const int kt_per = (KT + splits - 1) / splits;
      const int ns = (KT + kt_per - 1) / kt_per;  // every split gets at least one stage
      int32_t* acc32 = MODE == 0 ? acc : static_cast<int32_t*>(out);
      if (const hipError_t e = launch_zero32(acc32, M * N, s); e != hipSuccess) return e;
      const dim3 grid((unsigned)tiles, (unsigned)ns);
      if (K % BK == 0)
        hipLaunchKernelGGL((k_gemm<ABITS, BM, BN, WR, WC, BK, MODE, true, true>), grid, dim3(64 * WR * WC), 0, s,
                           codes, deq, Wq, w_scale, w_scale_up, (int)M, (int)N, (int)K, acc32, out, kt_per);
      else
        hipLaunchKernelGGL((k_gemm<ABITS, BM, BN, WR, WC, BK, MODE, false, true>), grid, dim3(64 * WR * WC), 0, s,
                           codes, deq, Wq, w_scale, w_scale_up, (int)M, (int)N, (int)K, acc32, out, kt_per);
      if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      if constexpr (MODE == 1) return launch_dequant32(out, deq, w_scale, M, N, s);
      return hipSuccess;
    }
  }
  if (K % BK == 0)
    hipLaunchKernelGGL((k_gemm<ABITS, BM, BN, WR, WC, BK, MODE, true, false>), dim3((unsigned)tiles),
                       dim3(64 * WR * WC), 0, s, codes, deq, Wq, w_scale, w_scale_up, (int)M, (int)N, (int)K, acc,
                       out, KT);
  else
    hipLaunchKernelGGL((k_gemm<ABITS, BM, BN, WR, WC, BK, MODE, false, false>), dim3((unsigned)tiles),
                       dim3(64 * WR * WC), 0, s, codes, deq, Wq, w_scale, w_scale_up, (int)M, (int)N, (int)K, acc,
                       out, KT);
  return hipGetLastError();
}

template <int ABITS, int MODE>
hipError_t launch(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale,
                  const float* w_scale_up, int64_t M, int64_t K, int64_t N, int32_t* acc, void* out, hipStream_t s) {
  constexpr int BKBIG = ABITS == 4 ? 256 : 128;  // INT8 A tiles are twice as wide in LDS
  if constexpr (MODE >= 2) {
    // The fused SwiGLU epilogue runs after the whole K, so the gate/up GEMM does not split;
    // with large problems it runs 128 x 256 tiles with four waves: two blocks share a CU and
    // one block's epilogue and start-up overlap the other's MFMAs.
    if (use_big_tiles(M, N)) {
      if (gemm_dma_ok(K, ABITS))
        return launch_gemm_dma(128, MODE, codes, deq, Wq, w_scale, w_scale_up, M, K, N, ABITS, acc, out, s);
      return launch_cfg<ABITS, 128, 256, 1, 4, BKBIG, MODE>(codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, 1,
                                                            s);
    }
    if (gemm_dma_ok(K, ABITS))
      return launch_gemm_dma(64, MODE, codes, deq, Wq, w_scale, w_scale_up, M, K, N, ABITS, acc, out, s);
    return launch_cfg<ABITS, 128, 128, 2, 2, 128, MODE>(codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, 1, s);
  } else {
    const GemmPlan p = plan_tiles(M, N, K);
    if (p.big && p.splits == 1 && gemm_dma_ok(K, ABITS))
      return launch_gemm_dma(256, MODE, codes, deq, Wq, w_scale, w_scale_up, M, K, N, ABITS, acc, out, s);
    if (p.big)
      return launch_cfg<ABITS, 256, 256, 2, 4, BKBIG, MODE>(codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out,
                                                            p.splits, s);
    if (small_tiles_unsplit(M, N, K) && gemm_dma_ok(K, ABITS))
      return launch_gemm_dma(64, MODE, codes, deq, Wq, w_scale, w_scale_up, M, K, N, ABITS, acc, out, s);
    return launch_cfg<ABITS, 128, 128, 2, 2, 128, MODE>(codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out,
                                                        p.splits, s);
  }
}

}  // namespace

// Tile choice: a 256x256 tile multiplies at roughly twice the rate of a 128x128 tile, so it
// wins unless it leaves most of the 256 CUs idle.
bool use_big_tiles(int64_t M, int64_t N) {
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const double time256 = (double)((t256 + CUS - 1) / CUS) * 4.0 / 2.0;
  const double time128 = (double)((t128 + CUS - 1) / CUS) * 1.0;
  return time256 <= time128;
}

// Below the 256 x 256 tiles, the 64 x 128 tiles of the LDS-direct kernel run unsplit when there
// are at least as many as CUs, or, for K up to 8192, a quarter of that: two or three of their
// blocks share a CU, where a 128 x 128 tile of four waves leaves one wave per SIMD.  Measured
// (a4 and a8, MI355X, with three stage buffers on the small tiles; four are a little faster
// again) against the 128 x 128 tiles with the K splits below: 2048^3 22 -> 16 us,
// M = 384 / 640 / 768 (N = 2048 ... 4096, K = 4096 ... 8192) 24 -> 14 us, 22 -> 13 us and
// 43 -> 31 us, M = 512, N = 4096, K = 16384 52 -> 39 us, M = 1000, N = 600, K = 8192 22.4 ->
// 20.9 us; below the thresholds the splits win (M = 256, N = 4096, K = 16384: 33.5 against
// 37.5 us; M = 128, N = 1024, K = 16384: 15 against 36 us).
bool small_tiles_unsplit(int64_t M, int64_t N, int64_t K) {
  const int64_t t64 = ((M + 63) / 64) * ((N + 127) / 128);
  return t64 >= CUS || (K <= 8192 && 4 * t64 >= CUS);
}

// Tiles and K splits for the product and dequant epilogues.  When the 256 x 256 tiles fill the
// CUs, or nearly (at least 192 tiles), they run unsplit.  Below that the 128 x 128 tiles run
// (several fit on a CU), and K may be split: the splits add their int32 results with atomics,
// whose cost grows with splits x M x N while each split's multiply time falls as K / splits, so
// the best count is about sqrt(1024 K / (M N)), taken to the nearest power of two (at most 8,
// at most two blocks per CU, each split at least 4 stages; no split below 2 when the tiles
// already fill the CUs).  Against a sweep of K = 2048 ... 16384, N = 4096, M = 65 ... 2048 over
// both tile sizes and 1 to 16 splits (a4, MI355X) this choice was the fastest or within 4 % of
// it at 26 of the 28 points, and within 13 % at all.
GemmPlan plan_tiles(int64_t M, int64_t N, int64_t K) {
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (t256 >= CUS) return GemmPlan{use_big_tiles(M, N), 1};
  if (t256 >= 3 * CUS / 4) return GemmPlan{true, 1};
  const double r = 0.5 * std::log2(1024.0 * (double)K / ((double)M * (double)N));
  int64_t splits = r <= 0.0 ? 1 : (int64_t)1 << std::min(3, (int)std::floor(r + 0.5));
  if (t128 >= CUS && r < 1.0) splits = 1;
  splits = std::min(splits, std::max<int64_t>(1, 2 * CUS / t128));
  splits = std::max<int64_t>(1, std::min(splits, ((K + 127) / 128) / 4));
  return GemmPlan{false, (int)splits};
}

// Zero n int32 (split-K accumulators; a kernel rather than a memset so that the sequence can
// be captured in a graph).
namespace {
__global__ __launch_bounds__(256) void k_zero32(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// In place: the int32 product acc[m, n] -> y[m, n] = fl(fl((float)acc * deq[m]) * alpha).
// Rows run over blockIdx.y and columns over blockIdx.x (grid-stride in both).
__global__ __launch_bounds__(256) void k_dequant32(void* __restrict__ buf, const float* __restrict__ deq,
                                                   const float* __restrict__ w_scale, int64_t M, int64_t N) {
  const float alpha = w_scale[0];
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const float dm = deq[m];
    const int32_t* acc = static_cast<const int32_t*>(buf) + m * N;
    float* y = static_cast<float*>(buf) + m * N;
    for (int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x; n < N; n += (int64_t)gridDim.x * 256)
      y[n] = __fmul_rn(__fmul_rn((float)acc[n], dm), alpha);
  }
}
}  // namespace

hipError_t launch_zero32(int32_t* p, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_zero32, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 2048)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_dequant32(void* buf, const float* deq, const float* w_scale, int64_t M, int64_t N, hipStream_t s) {
  hipLaunchKernelGGL(k_dequant32, dim3((unsigned)std::min<int64_t>((N + 255) / 256, 64), (unsigned)std::min<int64_t>(M, 1024)),
                     dim3(256), 0, s, buf, deq, w_scale, M, N);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale, int64_t M,
                       int64_t K, int64_t N, int abits, int32_t* acc, float* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (M <= GEMV_MAX_M) return launch_gemv(codes, deq, Wq, w_scale, M, K, N, abits, acc, y, s);
  if (acc != nullptr)
    return abits == 4 ? launch<4, 0>(codes, deq, Wq, w_scale, nullptr, M, K, N, acc, y, s)
                      : launch<8, 0>(codes, deq, Wq, w_scale, nullptr, M, K, N, acc, y, s);
  return abits == 4 ? launch<4, 1>(codes, deq, Wq, w_scale, nullptr, M, K, N, acc, y, s)
                    : launch<8, 1>(codes, deq, Wq, w_scale, nullptr, M, K, N, acc, y, s);
}

hipError_t launch_gemm_swiglu(const uint8_t* codes, const float* deq, const uint8_t* Wgu, const float* scale_gate,
                              const float* scale_up, int64_t M, int64_t K, int64_t F, int abits, int h_bf16, void* h,
                              hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t N = 2 * F;
  if (abits == 4)
    return h_bf16 ? launch<4, 3>(codes, deq, Wgu, scale_gate, scale_up, M, K, N, nullptr, h, s)
                  : launch<4, 2>(codes, deq, Wgu, scale_gate, scale_up, M, K, N, nullptr, h, s);
  return h_bf16 ? launch<8, 3>(codes, deq, Wgu, scale_gate, scale_up, M, K, N, nullptr, h, s)
                : launch<8, 2>(codes, deq, Wgu, scale_gate, scale_up, M, K, N, nullptr, h, s);
}

}  // namespace hbl
