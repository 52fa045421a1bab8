// k_gemm_f6f4.hip — the a4 GEMM on gfx950's scaled f8f6f4 matrix cores: INT4 activation
// codes stored as FP6 (E2M3) times ternary weights stored as FP4 (E2M1).
//
// The pages motivate 4-bit activations by hardware that computes natively in 4 bits
// (BitNet v2 write-up, section "原生4比特計算").  On MI355X the FP6/FP4 matrix path runs at
// twice the int8 rate.  Every INT4 code in [-7, 7] is exact in FP6 E2M3 and every ternary
// weight is exact in FP4 E2M1, each product is an integer of magnitude <= 7, and the fp32
// accumulator holds integer partial sums below 2^24 for K <= 2^21, so every sum is exact
// regardless of order: the result equals the int32 product bit for bit.  Block scales are
// fixed at 1 (E8M0 exponent 127).  No operand is decoded in this kernel; LDS fragments go
// straight into v_mfma_scale_f32_32x32x64_f8f6f4 (lane l: row / column l%32, the 32 k-values
// 32*(l/32) .. +31 of the 64-deep step; A as 6 registers of packed 6-bit codes, B as 4
// registers of packed nibbles).
//
// Tiling: a 512-thread block computes a 256 x 256 tile with 4 x 2 waves of 64 x 128 (128 fp32
// accumulators per lane, two waves per SIMD).  FP6/FP4 fragments are larger per MFMA than the
// int8 path's packed INT4/2-bit fragments (40 bytes per lane per 64-deep step), so LDS and L2
// traffic per MFMA is higher; the wave shape keeps A (the larger operand) read by only two
// waves.  K is staged through double-buffered LDS 128 deep.  A stage is short in time (two
// 64-deep MFMA steps), so global loads are issued two stages ahead into one of two register
// sets; with loads one stage ahead the waves waited on memory for most of each stage.  When
// K is a multiple of the stage depth the loads carry no K-tail masks.  See the main loop for
// the software pipeline.
#include <type_traits>

#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BK6 = 128;

__device__ __forceinline__ void tile_order(int bid, int nblk, int ntm, int ntn, int GM, int& tm, int& tn) {
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

// SPLIT: the block multiplies only the stages [blockIdx.y * kt_per, + kt_per) of K and adds
// its integer result into acc_out with atomics, as the int8 GEMM does for mid-size problems.
template <int BM, int BN, int WR, int WC, int MODE, bool FULLK, bool SPLIT>
__global__ __launch_bounds__(64 * WR * WC) void k_gemm_f6f4(const uint8_t* __restrict__ A,
                                                            const float* __restrict__ deq,
                                                            const uint8_t* __restrict__ B,
                                                            const float* __restrict__ w_scale, int M, int N, int K,
                                                            int32_t* __restrict__ acc_out, float* __restrict__ y,
                                                            int kt_per) {
  constexpr int NT = 64 * WR * WC;
  constexpr int KS = BK6 / 64;                // 64-deep MFMA steps per stage
  constexpr int AB = BK6 * 6 / 8;             // 96 bytes of FP6 codes per row per stage
  constexpr int AS = AB + 8;                  // 104: 26 dwords, distinct even banks for 16 rows
  constexpr int BB = BK6 / 2;                 // 64 bytes of FP4 weights per row per stage
  constexpr int BS = BB + 16;                 // 80: 20 dwords, distinct 4-bank groups for 8 rows
  constexpr int WM = BM / WR, WN = BN / WC;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int ACH = AB / 16, BCH = BB / 16;
  constexpr int ALD = BM * ACH / NT, BLD = BN * BCH / NT;
  static_assert(ALD * NT == BM * ACH && BLD * NT == BN * BCH, "tile/thread mismatch");
  static_assert(KS == 2, "the pipelined loop is written for two k-steps per stage");

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * AS];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * BS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WC, wn = wave % WC;
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  int tm, tn;
  tile_order(blockIdx.x, gridDim.x, ntm, ntn, 4, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t arow = (int64_t)K * 6 / 8;
  const int64_t brow = K / 2;
  const int KT = (K + BK6 - 1) / BK6;
  const int last_k64 = (K - (KT - 1) * BK6) / 64;
  const int kb = SPLIT ? (int)blockIdx.y * kt_per : 0;   // this block's first stage
  const int KTL = SPLIT ? min(KT - kb, kt_per) : KT;     // and its number of stages

  const uint8_t* Ablk = A + (int64_t)m0 * arow;
  const uint8_t* Bblk = B + (int64_t)n0 * brow;
  uint32_t aoff[ALD], boff[BLD];
#pragma unroll
  for (int i = 0; i < ALD; ++i) {
    const int e = tid + NT * i, r = e / ACH, c = e % ACH;
    aoff[i] = (uint32_t)(min(r, M - 1 - m0) * arow + 16 * c);
  }
#pragma unroll
  for (int i = 0; i < BLD; ++i) {
    const int e = tid + NT * i, r = e / BCH, c = e % BCH;
    boff[i] = (uint32_t)(min(r, N - 1 - n0) * brow + 16 * c);
  }

  // Two register sets stage the global loads: set S receives stage kt + 2 while the other set,
  // loaded a stage earlier, is stored to LDS.  S is a compile-time constant at every call;
  // the sets are chosen with if constexpr and copied element by element, because a run-time
  // subscript or pointer select on them makes the compiler keep them in memory (it then
  // moves them into LDS).
  struct Stage {
    uint4 a[ALD], b[BLD];
  };
  Stage st0, st1;
  auto stg = [&](auto S) __attribute__((always_inline)) -> Stage& {
    if constexpr (decltype(S)::value == 0) return st0;
    else return st1;
  };
  // Stage kt; in a partial last stage only the first n64 64-deep slices exist and the rest
  // is zero-filled (a zero FP4 weight contributes nothing).
  auto gload = [&](auto S, int kt, int n64) __attribute__((always_inline)) {
    Stage& r = stg(S);
    const uint8_t* ak = Ablk + (int64_t)kt * AB;
    const uint8_t* bk = Bblk + (int64_t)kt * BB;
    if constexpr (FULLK) {  // K a multiple of the stage depth: every chunk exists
#pragma unroll
      for (int i = 0; i < ALD; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(ak + aoff[i]);
        r.a[i] = make_uint4(v.x, v.y, v.z, v.w);
      }
#pragma unroll
      for (int i = 0; i < BLD; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(bk + boff[i]);
        r.b[i] = make_uint4(v.x, v.y, v.z, v.w);
      }
      return;
    }
    const int va = n64 * 48 / 16, vb = n64 * 32 / 16;
    // Chunks past the end are loaded from the last valid chunk of their row (always in
    // bounds) and cleared with a mask the compiler cannot see through, so the loads stay
    // unconditional and the loop body stays one basic block.
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int c = (tid + NT * i) % ACH, back = c < va ? 0 : 16 * (c - va + 1);
      uint32_t keep = c < va ? ~0u : 0u;
      asm volatile("" : "+v"(keep));
      const uint4 v = *reinterpret_cast<const uint4*>(ak + aoff[i] - back);
      r.a[i] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
      const int c = (tid + NT * i) % BCH, back = c < vb ? 0 : 16 * (c - vb + 1);
      uint32_t keep = c < vb ? ~0u : 0u;
      asm volatile("" : "+v"(keep));
      const uint4 v = *reinterpret_cast<const uint4*>(bk + boff[i] - back);
      r.b[i] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
    }
  };
  auto swrite = [&](auto S, int buf) __attribute__((always_inline)) {
    const Stage& r = stg(S);
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int e = tid + NT * i;
      uint8_t* d = &sA[buf][(e / ACH) * AS + 16 * (e % ACH)];
      reinterpret_cast<uint2*>(d)[0] = make_uint2(r.a[i].x, r.a[i].y);
      reinterpret_cast<uint2*>(d)[1] = make_uint2(r.a[i].z, r.a[i].w);
    }
#pragma unroll
    for (int i = 0; i < BLD; ++i) {
      const int e = tid + NT * i;
      *reinterpret_cast<uint4*>(&sB[buf][(e / BCH) * BS + 16 * (e % BCH)]) =
          make_uint4(r.b[i].x, r.b[i].y, r.b[i].z, r.b[i].w);
    }
  };

  struct Frag {
    uint2 a[TM][3];   // 24 bytes: 32 FP6 codes
    uint4 b[TN];      // 16 bytes: 32 FP4 weights
  };
  const int arow0 = (wm * WM + (lane & 31)) * AS + 24 * (lane >> 5);
  const int brow0 = (wn * WN + (lane & 31)) * BS + 16 * (lane >> 5);
  auto fread = [&](int buf, int ks, Frag& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint2* p = reinterpret_cast<const uint2*>(&sA[buf][arow0 + 32 * i * AS + ks * 48]);
      f.a[i][0] = p[0];
      f.a[i][1] = p[1];
      f.a[i][2] = p[2];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const uint4*>(&sB[buf][brow0 + 32 * j * BS + ks * 32]);
  };

  // Accumulators in the AGPR file (the "a" constraint selects the AGPR form of the MFMAs),
  // away from the VGPRs the loads and fragments use.
  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = v16f{};
      asm volatile("" : "+a"(acc[i][j]));
    }

  auto fmma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const v8i a = v8i{(int)f.a[i][0].x, (int)f.a[i][0].y, (int)f.a[i][1].x, (int)f.a[i][1].y,
                        (int)f.a[i][2].x, (int)f.a[i][2].y, 0, 0};
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v8i b = v8i{(int)f.b[j].x, (int)f.b[j].y, (int)f.b[j].z, (int)f.b[j].w, 0, 0, 0, 0};
        // cbsz = 2: A is FP6 E2M3; blgp = 4: B is FP4 E2M1; scales 127 = 2^0.
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 2, 4, 0, 127, 0, 127);
      }
    }
  };

  // Software pipeline over two LDS buffers and two register sets: the global loads of stage
  // kt + 2 are issued at the start of stage kt, and stage kt + 1 (loaded during stage kt - 1)
  // is stored into the other LDS buffer during kt's second k-step, so a load has about one
  // and a half stages to arrive; the fragments of each k-step are read during the MFMAs of
  // the previous one.  A stage has no branches (loads past the last stage reload the last
  // one, and what they store goes to the idle buffer), so it is one scheduling region, and
  // the group barriers interleave one memory instruction after each MFMA.  Two waves share
  // each SIMD, so one wave's barrier or load wait is covered by the other's MFMAs.
  constexpr int NMF = TM * TN;                 // MFMAs per k-step
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  Frag f0, f1;
  // One stage; S is the register set that receives stage kt + 2.
  auto stage = [&](auto S, int kt) __attribute__((always_inline)) {
    constexpr int set = decltype(S)::value;
    const int buf = kt & 1;
    const int nx = kb + min(kt + 2, KTL - 1);  // kt counts this block's stages
    gload(S, nx, nx == KT - 1 ? last_k64 : KS);
    fread(buf, 1, f1);
    fmma(f0);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      if (i < ALD + BLD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    swrite(std::integral_constant<int, 1 - set>{}, buf ^ 1);
    fmma(f1);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // one LDS write
    }
    __syncthreads();
    fread(buf ^ 1, 0, f0);
  };
  gload(I0{}, kb, kb == KT - 1 ? last_k64 : KS);
  const int n1 = kb + min(1, KTL - 1);
  gload(I1{}, n1, n1 == KT - 1 ? last_k64 : KS);
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
        const float a = acc[i][j][v];  // an exact integer
        if constexpr (SPLIT) {
          atomicAdd(&acc_out[(int64_t)m * N + n], (int32_t)a);
        } else if constexpr (MODE == 0) {
          acc_out[(int64_t)m * N + n] = (int32_t)a;
        } else {
          y[(int64_t)m * N + n] = __fmul_rn(__fmul_rn(a, dm), alpha);
        }
      }
    }
  }
}

// The same product with its tiles loaded straight into LDS (buffer_load_dwordx4 ... lds, as
// in k_gemm_dma.hip), for 256 x 256 tiles and K a multiple of the 128-deep stage: no register
// set stages the tiles and no ds_write stores them.  Three stage buffers of 40 KB; a stage's
// loads are issued right after the barrier in the middle of the stage NBUF earlier and waited
// for at the barrier in the middle of the stage before it.
//
// k permutation.  The matrix core takes any assignment of k to (lane half, position) as long
// as A and B use the same, and every sum here is exact in any order.  In a stage, lane half h
// of k-step t multiplies codes 64 h + 32 t + 0..31 of the stage: its A operands for both steps
// are then the 48 contiguous bytes of codes 64 h .. 64 h + 63 (three 16-byte chunks, read with
// 128-bit LDS reads; step 0 takes the first 24 bytes, step 1 the last 24) and its B operands
// the 16-byte chunks 2 h and 2 h + 1 of the row's 64 weight bytes.
//
// LDS slots (16 bytes): A row r holds 6 chunks at slots 6 r + (c ^ ((r >> 3) & 1)), B row n 4
// chunks at 4 n + (c ^ ((n >> 2) & 3)).  The 16 lanes of a 128-bit read pass (16 consecutive
// rows, one chunk) then hit 16 different bank groups: 6 r mod 16 runs over the even values
// twice (r and r + 8), and the XOR gives those two rows chunks of opposite parity.
template <int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_f6f4_dma(
    const uint8_t* __restrict__ A, const float* __restrict__ deq, const uint8_t* __restrict__ B,
    const float* __restrict__ w_scale, int M, int N, int K, int32_t* __restrict__ acc_out, float* __restrict__ y) {
  constexpr int BM = 256, BN = 256, WR = 4, WC = 2, NW = WR * WC, NBUF = 3;
  constexpr int AB = BK6 * 6 / 8, BB = BK6 / 2;   // 96 and 64 bytes per row per stage
  constexpr int A_BYTES = BM * AB, B_BYTES = BN * BB, STAGE = A_BYTES + B_BYTES;
  constexpr int AI = BM * 6 / 64 / NW, BI = BN * 4 / 64 / NW;   // load instructions per wave per stage
  constexpr int WM = BM / WR, WN = BN / WC, TM = WM / 32, TN = WN / 32;
  static_assert(AI * 64 * NW == BM * 6 && BI * 64 * NW == BN * 4, "load instructions per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WC, wn = wave % WC;
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  int tm, tn;
  tile_order(blockIdx.x, gridDim.x, ntm, ntn, 4, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t arow = (int64_t)K * 6 / 8, brow = K / 2;
  const int KT = K / BK6;

  const v4u_t rA = buffer_rsrc(A + (int64_t)m0 * arow, (uint32_t)(min(BM, M - m0) * arow));
  const v4u_t rB = buffer_rsrc(B + (int64_t)n0 * brow, (uint32_t)(min(BN, N - n0) * brow));
  uint32_t aoff[AI], boff[BI];   // rows past M (N) re-read the last row
#pragma unroll
  for (int a = 0; a < AI; ++a) {
    const int sl = 64 * (wave * AI + a) + lane, r = sl / 6, c = (sl % 6) ^ ((r >> 3) & 1);
    aoff[a] = (uint32_t)(min(r, M - 1 - m0) * arow + 16 * c);
  }
#pragma unroll
  for (int b = 0; b < BI; ++b) {
    const int sl = 64 * (wave * BI + b) + lane, n = sl / 4, c = (sl % 4) ^ ((n >> 2) & 3);
    boff[b] = (uint32_t)(min(n, N - 1 - n0) * brow + 16 * c);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto load_stage = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t sa = lds0 + buf * STAGE, sb = sa + A_BYTES;
#pragma unroll
    for (int a = 0; a < AI; ++a) dma16(rA, aoff[a], kt * AB, sa + 1024 * (wave * AI + a));
#pragma unroll
    for (int b = 0; b < BI; ++b) dma16(rB, boff[b], kt * BB, sb + 1024 * (wave * BI + b));
  };

  // fragment addresses within a stage buffer (rows l % 32 of the wave's tiles; half h = l / 32)
  const int l32 = lane & 31, h = lane >> 5;
  int afr[3], bfr[2];
#pragma unroll
  for (int e = 0; e < 3; ++e) afr[e] = 16 * (6 * (wm * WM + l32) + ((3 * h + e) ^ ((l32 >> 3) & 1)));
#pragma unroll
  for (int t = 0; t < 2; ++t) bfr[t] = A_BYTES + 16 * (4 * (wn * WN + l32) + ((2 * h + t) ^ ((l32 >> 2) & 3)));
  // part 0 (k-step 0): A chunks 0, 1 and B chunk 0; part 1 (k-step 1): the upper half of A
  // chunk 1 (kept from part 0), A chunk 2 and B chunk 1
  typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
  struct F0 {
    v4u_t a[TM][2];
    v4u_t b[TN];
  };
  struct F1 {
    v2u_t hi[TM];
    v4u_t a[TM];
    v4u_t b[TN];
  };
  auto read0 = [&](int buf, F0& f) __attribute__((always_inline)) {
    const uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 2; ++e) f.a[i][e] = *reinterpret_cast<const v4u_t*>(base + afr[e] + 32 * 6 * 16 * i);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const v4u_t*>(base + bfr[0] + 32 * 4 * 16 * j);
  };
  auto read1 = [&](int buf, F1& f) __attribute__((always_inline)) {
    const uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const v4u_t*>(base + afr[2] + 32 * 6 * 16 * i);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const v4u_t*>(base + bfr[1] + 32 * 4 * 16 * j);
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = v16f{};
      asm volatile("" : "+a"(acc[i][j]));
    }
  auto mma0 = [&](const F0& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const v8i a = v8i{(int)f.a[i][0].x, (int)f.a[i][0].y, (int)f.a[i][0].z, (int)f.a[i][0].w,
                        (int)f.a[i][1].x, (int)f.a[i][1].y, 0, 0};
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v8i b = v8i{(int)f.b[j].x, (int)f.b[j].y, (int)f.b[j].z, (int)f.b[j].w, 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 2, 4, 0, 127, 0, 127);
      }
    }
  };
  auto mma1 = [&](const F1& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const v8i a = v8i{(int)f.hi[i].x, (int)f.hi[i].y, (int)f.a[i].x, (int)f.a[i].y, (int)f.a[i].z, (int)f.a[i].w,
                        0, 0};
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v8i b = v8i{(int)f.b[j].x, (int)f.b[j].y, (int)f.b[j].z, (int)f.b[j].w, 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 2, 4, 0, 127, 0, 127);
      }
    }
  };

  // Pipeline as in k_gemm_dma.hip: stage s in buffer s % NBUF, its loads issued after the
  // middle barrier of stage s - NBUF and complete at the middle barrier of stage s - 1; past
  // the last stage the last one is loaded again into a buffer no one reads.
  constexpr int PER_STAGE = AI + BI;
#pragma unroll
  for (int st = 0; st < NBUF; ++st) load_stage(min(st, KT - 1), st);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 1) * PER_STAGE) : "memory");
  __syncthreads();
  F0 f0;
  F1 f1;
  read0(0, f0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt % NBUF;
    read1(buf, f1);
#pragma unroll
    for (int i = 0; i < TM; ++i) f1.hi[i] = v2u_t{f0.a[i][1].z, f0.a[i][1].w};
    mma0(f0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 2) * PER_STAGE) : "memory");
    __syncthreads();
    load_stage(min(kt + NBUF, KT - 1), buf);
    read0((kt + 1) % NBUF, f0);
    mma1(f1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still write LDS

  // Epilogue through LDS as in k_gemm_dma.hip: one 32-row MFMA tile row and half of the wave's
  // columns (64) at a time, each wave in a region of its own ([32][72] words) inside the stage
  // buffers, so that every store writes 16 contiguous bytes per lane.
  __syncthreads();
  const int el = __lane_id();
  const int col = el & 31, rh = 4 * (el >> 5);
  constexpr int S = 64 + 8;   // 4 S = 32 modulo the 64 banks
  static_assert(NW * 32 * S * 4 <= NBUF * STAGE, "the staging regions fit the stage buffers");
  uint32_t* stg = reinterpret_cast<uint32_t*>(lds) + wave * 32 * S;
  float alpha = 0.0f;
  if constexpr (MODE == 1) alpha = w_scale[0];
  uint32_t* dst = MODE == 0 ? reinterpret_cast<uint32_t*>(acc_out) : reinterpret_cast<uint32_t*>(y);
  const int mw = m0 + wm * WM;
  const bool vec = (N & 3) == 0;   // rows start 16-byte aligned
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int hj = 0; hj < TN / 2; ++hj) {
      // the accumulators of this piece are read only from here on
      asm volatile("" : "+a"(acc[i][2 * hj]), "+a"(acc[i][2 * hj + 1]));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + rh + (v & 3);
        const int m = mw + 32 * i + r;
        float dm = 0.0f;
        if constexpr (MODE == 1) dm = m < M ? deq[m] : 0.0f;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const float a = acc[i][2 * hj + jj][v];  // an exact integer
          stg[r * S + 32 * jj + col] =
              MODE == 0 ? (uint32_t)(int32_t)a : __float_as_uint(__fmul_rn(__fmul_rn(a, dm), alpha));
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int r = (el >> 4) + 4 * p, c = el & 15;
        const int m = mw + 32 * i + r, n = n0 + wn * WN + 64 * hj + 4 * c;
        const uint4 q = *reinterpret_cast<const uint4*>(stg + r * S + 4 * c);
        if (m >= M || n >= N) continue;
        uint32_t* yp = dst + (int64_t)m * N + n;
        if (vec && n + 3 < N) {
          *reinterpret_cast<uint4*>(yp) = q;
        } else {
          yp[0] = q.x;
          if (n + 1 < N) yp[1] = q.y;
          if (n + 2 < N) yp[2] = q.z;
          if (n + 3 < N) yp[3] = q.w;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the next piece is staged
    }
  }
}

template <int BM, int BN, int WR, int WC, int MODE>
hipError_t launch_cfg(const uint8_t* codes, const float* deq, const uint8_t* Wq4, const float* w_scale, int64_t M,
                      int64_t K, int64_t N, int32_t* acc, float* y, int splits, hipStream_t s) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int KT = (int)((K + BK6 - 1) / BK6);
  if (splits > 1) {
    const int kt_per = (KT + splits - 1) / splits;
    const int ns = (KT + kt_per - 1) / kt_per;  // every split gets at least one stage
    int32_t* acc32 = MODE == 0 ? acc : reinterpret_cast<int32_t*>(y);
    if (const hipError_t e = launch_zero32(acc32, M * N, s); e != hipSuccess) return e;
    const dim3 grid((unsigned)tiles, (unsigned)ns);
    if (K % BK6 == 0)
      hipLaunchKernelGGL((k_gemm_f6f4<BM, BN, WR, WC, MODE, true, true>), grid, dim3(64 * WR * WC), 0, s, codes, deq,
                         Wq4, w_scale, (int)M, (int)N, (int)K, acc32, y, kt_per);
    else
      hipLaunchKernelGGL((k_gemm_f6f4<BM, BN, WR, WC, MODE, false, true>), grid, dim3(64 * WR * WC), 0, s, codes, deq,
                         Wq4, w_scale, (int)M, (int)N, (int)K, acc32, y, kt_per);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if constexpr (MODE == 1) return launch_dequant32(y, deq, w_scale, M, N, s);
    return hipSuccess;
  }
  if (K % BK6 == 0)
    hipLaunchKernelGGL((k_gemm_f6f4<BM, BN, WR, WC, MODE, true, false>), dim3((unsigned)tiles), dim3(64 * WR * WC), 0,
                       s, codes, deq, Wq4, w_scale, (int)M, (int)N, (int)K, acc, y, KT);
  else
    hipLaunchKernelGGL((k_gemm_f6f4<BM, BN, WR, WC, MODE, false, false>), dim3((unsigned)tiles), dim3(64 * WR * WC), 0,
                       s, codes, deq, Wq4, w_scale, (int)M, (int)N, (int)K, acc, y, KT);
  return hipGetLastError();
}

// The tile size and K splits follow the int8 GEMM's plan (plan_tiles): 256 x 256 tiles when
// they (nearly) fill the CUs, else 128 x 128 tiles with K split when those are few.
template <int MODE>
hipError_t launch(const uint8_t* codes, const float* deq, const uint8_t* Wq4, const float* w_scale, int64_t M,
                  int64_t K, int64_t N, int32_t* acc, float* y, hipStream_t s) {
  const GemmPlan p = plan_tiles(M, N, K);
  if (p.big && p.splits == 1 && K % BK6 == 0) {
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    hipLaunchKernelGGL((k_gemm_f6f4_dma<MODE>), dim3((unsigned)tiles), dim3(512), 0, s, codes, deq, Wq4, w_scale,
                       (int)M, (int)N, (int)K, acc, y);
    return hipGetLastError();
  }
  if (p.big) return launch_cfg<256, 256, 4, 2, MODE>(codes, deq, Wq4, w_scale, M, K, N, acc, y, p.splits, s);
  return launch_cfg<128, 128, 2, 2, MODE>(codes, deq, Wq4, w_scale, M, K, N, acc, y, p.splits, s);
}

// Ternary 2-bit words (16 weights, weight c in field 4(c%4)+c/4) -> FP4 E2M1 nibbles in
// natural order (weight c in nibble c): 0 -> 0x0, +1 -> 0x2 (1.0), -1 -> 0xA (-1.0).
__global__ __launch_bounds__(256) void k_weights_fp4(const uint32_t* __restrict__ Wq, int64_t words,
                                                     uint2* __restrict__ Wq4) {
  for (int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x; w < words; w += (int64_t)gridDim.x * 256) {
    const uint32_t src = Wq[w];
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint32_t f = (src >> (2 * (4 * (c & 3) + (c >> 2)))) & 3u;  // 00 = 0, 01 = +1, 11 = -1
      const uint32_t nib = f == 1u ? 0x2u : (f == 3u ? 0xAu : 0x0u);
      if (c < 8) lo |= nib << (4 * c);
      else hi |= nib << (4 * (c - 8));
    }
    Wq4[w] = make_uint2(lo, hi);
  }
}

}  // namespace

hipError_t launch_gemm_f6f4(const uint8_t* codes6, const float* deq, const uint8_t* Wq4, const float* w_scale,
                            int64_t M, int64_t K, int64_t N, int32_t* acc, float* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (acc != nullptr) return launch<0>(codes6, deq, Wq4, w_scale, M, K, N, acc, y, s);
  return launch<1>(codes6, deq, Wq4, w_scale, M, K, N, acc, y, s);
}

hipError_t launch_weights_fp4(const uint8_t* Wq, int64_t N, int64_t K, uint8_t* Wq4, hipStream_t s) {
  const int64_t words = N * K / 16;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_weights_fp4, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const uint32_t*>(Wq),
                     words, reinterpret_cast<uint2*>(Wq4));
  return hipGetLastError();
}

}  // namespace hbl
