// k_gemm_dma.hip — the ternary x INT4/INT8 GEMM of k_gemm.hip with its operand tiles moved from
// global memory straight into LDS by the buffer loads' LDS mode (buffer_load_dwordx4 ... lds),
// for problems whose K is a multiple of the stage depth.
//
// BitNet v2 write-up, section H-BitLinear模塊: the quantised activations multiply the ternary
// weights and the result is rescaled by the activation and weight scales (bitnet.cpp article:
// with weights in {-1, 0, 1} the product needs only additions).  As in k_gemm.hip the codes and
// weights are widened to int8 in registers and multiplied on v_mfma_i32_32x32x32_i8; the int32
// sums, and so every output, are identical.
//
// What changes is the staging.  A load instruction of a wave writes its 64 lanes' 16 bytes to 64
// consecutive 16-byte LDS slots, so no register holds the tile on its way and no ds_write
// moves it; a stage's tiles are in flight while the previous stages are multiplied (NBUF LDS
// buffers, one barrier per stage).  Since a lane may load any 16 bytes, the assignment of
// (row, chunk) pairs to slots is free: within a row the 16-byte chunks are XOR-swizzled by row
// bits, so that the fragment reads below hit 16 different bank groups in each 16-lane pass of a
// 128-bit LDS read (64 banks of 4 bytes).
//
// Fragments are read 128 bits at a time, four 32-deep k-steps ("a quad") at once.  The
// matrix core takes any assignment of k to (lane half, byte) as long as A and B use the same:
// over a quad of 128 k-values, lane half h of step t multiplies the 16 k-values of weight word
// 4h + t of the quad, i.e. codes 32 (2h + t/2) + 16 (t%2) + 0..15.  Then a lane's B operands of
// the quad are one 16-byte slot (four weight words) and its INT4 A operands two slots (INT8: four).
#include <type_traits>

#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

// Block-to-tile order as in k_gemm.hip: every XCD gets a contiguous chunk of tile ids, which
// advance over groups of GM tile-rows.
__device__ __forceinline__ void dma_tile_of_block(int bid, int nblk, int ntm, int ntn, int GM, int& tm, int& tn) {
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

// Slot swizzles (16-byte units).  A rows hold 8 slots per stage: chunk c of row r sits in slot
// c ^ ((r >> 1) & 7).  B rows hold 4 slots (INT4 stages, 256 k) or 2 (INT8, 128 k): slot s of
// row n in s ^ ((n >> 2) & 3), resp. s ^ ((n >> 3) & 1).
__device__ __forceinline__ constexpr int swz_a(int r) { return (r >> 1) & 7; }
template <int ABITS>
__device__ __forceinline__ constexpr int swz_b(int n) { return ABITS == 4 ? (n >> 2) & 3 : (n >> 3) & 1; }

template <int ABITS, int BM, int BN, int WR, int WC, int MODE, int NBUF>
__global__ __launch_bounds__(64 * WR * WC) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_dma(
    const uint8_t* __restrict__ A, const float* __restrict__ deq, const uint8_t* __restrict__ B,
    const float* __restrict__ w_scale, const float* __restrict__ w_scale_up, int M, int N, int K,
    int32_t* __restrict__ acc_out, void* __restrict__ out) {
  constexpr int NW = WR * WC;
  constexpr int BK = ABITS == 4 ? 256 : 128;        // k per stage
  constexpr int AB = BK * ABITS / 8;                // A bytes per row per stage (128)
  constexpr int BB = BK / 4;                        // B bytes per row per stage (64 / 32)
  constexpr int BSL = BB / 16;                      // B slots per row per stage (4 / 2)
  constexpr int QUADS = BK / 128;                   // quads per stage (2 / 1)
  constexpr int A_BYTES = BM * AB, B_BYTES = BN * BB;
  constexpr int AI = BM * 8 / 64 / NW;              // A load instructions per wave per stage
  constexpr int BI = BN * BSL / 64 / NW;            // B load instructions per wave per stage
  constexpr int WM = BM / WR, WN = BN / WC;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int SHIFT = ABITS == 4 ? 10 : 6;
  static_assert(AB == 128, "8 A slots per row per stage");
  static_assert(AI * NW * 64 == BM * 8 && BI * NW * 64 == BN * BSL, "load instructions per wave");
  static_assert(TN % 2 == 0, "weight words of tile pairs are widened together");
  static_assert(MODE < 2 || WN == 64, "the fused gate/up epilogue pairs a wave's two 32-column tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * (A_BYTES + B_BYTES)];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WC, wn = wave % WC;
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  // Tile-rows per group: the 32 CUs of an XCD work on GM tile-rows at once, and the operand
  // slices those tiles stream should fit its 4 MB L2.  256 x 256 tiles (one per CU): 4 rows x 8
  // columns.  128 x 256 tiles (the gate/up GEMM, two per CU): 8 rows x 8 columns, 2 MB of codes
  // and 2 MB of weights over K = 4096, where 4 x 16 streamed 5 MB (632 -> 520 MB fetched from
  // beyond L2 per 7B gate/up launch).
  constexpr int GM = BM == 128 ? 8 : 4;
  int tm, tn;
  dma_tile_of_block(blockIdx.x, gridDim.x, ntm, ntn, GM, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t arow = (int64_t)K * ABITS / 8;
  const int64_t brow = K / 4;
  const int KT = K / BK;

  // Loads: instruction a of this wave fills A slots [64 (wave AI + a), +64); lane l takes slot
  // 64 (wave AI + a) + l, i.e. row 8 (wave AI + a) + l / 8 and physical chunk l % 8, whose
  // logical chunk is the swizzled one.  Rows past M (columns past N) are clamped.
  const v4u_t rA = buffer_rsrc(A + (int64_t)m0 * arow, (uint32_t)(min(BM, M - m0) * arow));
  const v4u_t rB = buffer_rsrc(B + (int64_t)n0 * brow, (uint32_t)(min(BN, N - n0) * brow));
  uint32_t aoff[AI], boff[BI];
#pragma unroll
  for (int a = 0; a < AI; ++a) {
    const int r = 8 * (wave * AI + a) + (lane >> 3);
    aoff[a] = (uint32_t)(min(r, M - 1 - m0) * arow + 16 * ((lane & 7) ^ swz_a(r)));
  }
#pragma unroll
  for (int b = 0; b < BI; ++b) {
    const int n = (64 / BSL) * (wave * BI + b) + lane / BSL;
    boff[b] = (uint32_t)(min(n, N - 1 - n0) * brow + 16 * ((lane % BSL) ^ swz_b<ABITS>(n)));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto load_stage = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t sa = lds0 + buf * (A_BYTES + B_BYTES), sb = sa + A_BYTES;
#pragma unroll
    for (int a = 0; a < AI; ++a) dma16(rA, aoff[a], kt * AB, sa + 1024 * (wave * AI + a));
#pragma unroll
    for (int b = 0; b < BI; ++b) dma16(rB, boff[b], kt * BB, sb + 1024 * (wave * BI + b));
  };

  // Fragment addresses (bytes, within a stage buffer).  Lane l reads rows / columns l % 32 of its
  // wave's 32-row / 32-column tiles; half h = l / 32.  The swizzle of those rows depends only on
  // l % 32 (tile bases are multiples of 32).  A stage is multiplied in two parts, each from two
  // A slots and one B slot per tile and lane: INT4, part p is quad p (codes 128 p + 16 (4 h + t)
  // + 0..15 at step t = 0..3); INT8, part p is steps 2p and 2p + 1 of the stage's one quad (codes
  // 16 (4 h + t) + 0..15), both parts reading the same B slot.
  const int l32 = lane & 31, h = lane >> 5;
  int afr[2][2], bfr[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = ABITS == 4 ? 4 * p + 2 * h + e : 4 * h + 2 * p + e;   // logical chunk
      afr[p][e] = (wm * WM + l32) * AB + 16 * (c ^ swz_a(l32));
    }
    const int sl = ABITS == 4 ? 2 * p + h : h;   // logical B slot
    bfr[p] = A_BYTES + (wn * WN + l32) * BB + 16 * (sl ^ swz_b<ABITS>(l32));
  }

  struct Frag {
    uint4 a[TM][2];
    uint4 b[TN];
  };
  auto fread = [&](int buf, int p, Frag& f) __attribute__((always_inline)) {
    const uint8_t* base = lds + buf * (A_BYTES + B_BYTES);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 2; ++e) f.a[i][e] = *reinterpret_cast<const uint4*>(base + afr[p][e] + 32 * AB * i);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const uint4*>(base + bfr[p] + 32 * BB * j);
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = v16i{};
      asm volatile("" : "+a"(acc[i][j]));
    }

  // The MFMAs of part p: at each step, B word t of each column tile widened to 64 t (pairs of
  // tiles with 64-bit shifts, as in k_gemm.hip), the A codes of the step widened to 16 q (INT4)
  // or taken as they are.
  auto part_mma = [&](const Frag& f, const int p) __attribute__((always_inline)) {
    constexpr int STEPS = ABITS == 4 ? 4 : 2;
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const int t = ABITS == 4 ? u : 2 * p + u;   // B word of the step
      v4i bo[TN];
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const uint32_t w0 = t == 0 ? f.b[j].x : t == 1 ? f.b[j].y : t == 2 ? f.b[j].z : f.b[j].w;
        const uint32_t w1 = t == 0 ? f.b[j + 1].x : t == 1 ? f.b[j + 1].y : t == 2 ? f.b[j + 1].z : f.b[j + 1].w;
        const uint64_t w = (uint64_t)w0 | ((uint64_t)w1 << 32);
        uint64_t w6 = w << 6, w4 = w << 4, w2 = w << 2;
        asm volatile("" : "+v"(w6), "+v"(w4), "+v"(w2));  // keep each shift one 64-bit op
        bo[j] = v4i{(int)((uint32_t)w6 & 0xC0C0C0C0u), (int)((uint32_t)w4 & 0xC0C0C0C0u),
                    (int)((uint32_t)w2 & 0xC0C0C0C0u), (int)((uint32_t)w & 0xC0C0C0C0u)};
        bo[j + 1] = v4i{(int)((uint32_t)(w6 >> 32) & 0xC0C0C0C0u), (int)((uint32_t)(w4 >> 32) & 0xC0C0C0C0u),
                        (int)((uint32_t)(w2 >> 32) & 0xC0C0C0C0u), (int)((uint32_t)(w >> 32) & 0xC0C0C0C0u)};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        v4i ao;
        if constexpr (ABITS == 4) {
          const uint4 c = f.a[i][u >> 1];
          const uint64_t w = (u & 1) ? ((uint64_t)c.z | ((uint64_t)c.w << 32)) : ((uint64_t)c.x | ((uint64_t)c.y << 32));
          uint64_t w4 = w << 4;
          asm volatile("" : "+v"(w4));
          ao = v4i{(int)((uint32_t)w4 & 0xF0F0F0F0u), (int)((uint32_t)w & 0xF0F0F0F0u),
                   (int)((uint32_t)(w4 >> 32) & 0xF0F0F0F0u), (int)((uint32_t)(w >> 32) & 0xF0F0F0F0u)};
        } else {
          const uint4 c = f.a[i][u];
          ao = v4i{(int)c.x, (int)c.y, (int)c.z, (int)c.w};
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao, bo[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // Pipeline.  Stage s goes to buffer s % NBUF; its loads are issued once no wave reads that
  // buffer any more, i.e. right after the barrier in the middle of stage s - NBUF, and must be
  // complete at the barrier in the middle of stage s - 1, after which its part 0 is read.  So the
  // loads have NBUF - 1 stages of MFMA work to arrive, and the one barrier per stage sits
  // between the two parts, with part 1's fragments already in registers: no wave waits for an
  // LDS read after it.  Past the last stage the last one is loaded again (into a buffer no one
  // reads), so that every stage issues the same loads and the counter waits stay exact.
  constexpr int PER_STAGE = AI + BI;                 // load instructions per wave per stage
#pragma unroll
  for (int st = 0; st < NBUF; ++st) load_stage(min(st, KT - 1), st);
  // stage 0 complete: the NBUF - 1 younger stages may still be in flight
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 1) * PER_STAGE) : "memory");
  __syncthreads();
  Frag f0, f1;
  fread(0, 0, f0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt % NBUF;
    fread(buf, 1, f1);
    part_mma(f0, 0);
    // this wave's reads of buffer `buf` have returned, and stage kt + 1 has arrived (only the
    // NBUF - 2 younger stages may be pending)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 2) * PER_STAGE) : "memory");
    __syncthreads();
    load_stage(min(kt + NBUF, KT - 1), buf);
    fread((kt + 1) % NBUF, 0, f0);
    part_mma(f1, 1);
  }
  // no load may still be writing this block's LDS when its waves end
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue.  The outputs are computed as in k_gemm.hip, then passed through LDS one 32-row
  // MFMA tile row at a time, so that every store writes 16 contiguous bytes per lane (a wave's
  // row segment of 64 outputs, or of 32 h values, in 16-byte pieces) instead of one element per
  // lane scattered over two rows.  Each wave stages in a region of its own ([32][S] words; 4 S
  // is 32 modulo the 64 banks, so the two half-waves' writes of one tile row hit different
  // banks) inside the stage buffers, which no load writes any more once every wave has waited
  // for its loads and passed the barrier.
  __syncthreads();
  const int el = __lane_id();
  const int col = el & 31, rh = 4 * (el >> 5);   // accumulator column and row offset of this lane
  constexpr int W = MODE >= 2 ? 32 : WN;         // outputs per row of the wave's tile
  constexpr int S = W + 8;
  static_assert(NW * 32 * S * 4 <= NBUF * (A_BYTES + B_BYTES), "the staging regions fit the stage buffers");
  uint32_t* stg = reinterpret_cast<uint32_t*>(lds) + wave * 32 * S;
  const int mw = m0 + wm * WM;                   // first row of this wave's tile
  if constexpr (MODE >= 2) {
    const float ag = w_scale[0], au = w_scale_up[0];
    const int F = N / 2;
    const int nb = n0 / 2 + wn * 32;             // first h column of the wave (F % 32 == 0)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      // the accumulators of tile row i are read only from here on
      asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + rh + (v & 3);
        const int m = mw + 32 * i + r;
        float hh = 0.0f;
        if (m < M) {
          const float dm = deq[m];
          const float g = __fmul_rn(__fmul_rn((float)(acc[i][0][v] >> SHIFT), dm), ag);
          const float u = __fmul_rn(__fmul_rn((float)(acc[i][1][v] >> SHIFT), dm), au);
          hh = silu_mul(g, u);
        }
        stg[r * S + col] = __float_as_uint(hh);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (MODE == 3) {
        // lane: 8 consecutive h values of one row -> 16 bytes of bf16
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int r = (el >> 2) + 16 * p, o = el & 3;
          const int m = mw + 32 * i + r;
          const uint4 a = *reinterpret_cast<const uint4*>(stg + r * S + 8 * o);
          const uint4 b = *reinterpret_cast<const uint4*>(stg + r * S + 8 * o + 4);
          if (m < M && nb < F) {
            const uint4 q = make_uint4(bf16x2_rne(a.x, a.y), bf16x2_rne(a.z, a.w), bf16x2_rne(b.x, b.y),
                                       bf16x2_rne(b.z, b.w));
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + (int64_t)m * F + nb + 8 * o) = q;
          }
        }
      } else {
        // lane: 4 consecutive h values of one row -> 16 bytes of fp32
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int r = (el >> 3) + 8 * p, c = el & 7;
          const int m = mw + 32 * i + r;
          const uint4 q = *reinterpret_cast<const uint4*>(stg + r * S + 4 * c);
          if (m < M && nb < F) *reinterpret_cast<uint4*>(static_cast<float*>(out) + (int64_t)m * F + nb + 4 * c) = q;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the next tile row is staged
    }
    return;
  }
  float alpha = 0.0f;
  if constexpr (MODE == 1) alpha = w_scale[0];
  uint32_t* dst = MODE == 0 ? reinterpret_cast<uint32_t*>(acc_out) : static_cast<uint32_t*>(out);
  const int nb = n0 + wn * WN;                   // first column of this wave
  const bool vec = (N & 3) == 0;                 // rows start 16-byte aligned
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    // the accumulators of tile row i are read only from here on (otherwise the compiler moves
    // all of them to VGPRs at once and spills)
#pragma unroll
    for (int j = 0; j < TN; ++j) asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + rh + (v & 3);
      const int m = mw + 32 * i + r;
      float dm = 0.0f;
      if constexpr (MODE == 1) dm = m < M ? deq[m] : 0.0f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int val = acc[i][j][v] >> SHIFT;
        stg[r * S + 32 * j + col] =
            MODE == 0 ? (uint32_t)val : __float_as_uint(__fmul_rn(__fmul_rn((float)val, dm), alpha));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // lane: 4 consecutive outputs of one row -> 16 bytes
#pragma unroll
    for (int p = 0; p < 32 * WN / 4 / 64; ++p) {
      const int r = (el >> 4) + 4 * p, c = el & 15;
      const int m = mw + 32 * i + r, n = nb + 4 * c;
      const uint4 q = *reinterpret_cast<const uint4*>(stg + r * S + 4 * c);
      if (m >= M || n >= N) continue;
      uint32_t* y = dst + (int64_t)m * N + n;
      if (vec && n + 3 < N) {
        *reinterpret_cast<uint4*>(y) = q;
      } else {
        y[0] = q.x;
        if (n + 1 < N) y[1] = q.y;
        if (n + 2 < N) y[2] = q.z;
        if (n + 3 < N) y[3] = q.w;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the next tile row is staged
  }
}

template <int ABITS, int BM, int BN, int WR, int WC, int MODE, int NBUF>
hipError_t launch_dma_cfg(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale,
                          const float* w_scale_up, int64_t M, int64_t K, int64_t N, int32_t* acc, void* out,
                          hipStream_t s) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm_dma<ABITS, BM, BN, WR, WC, MODE, NBUF>), dim3((unsigned)tiles), dim3(64 * WR * WC), 0, s,
                     codes, deq, Wq, w_scale, w_scale_up, (int)M, (int)N, (int)K, acc, out);
  return hipGetLastError();
}

template <int ABITS, int MODE>
hipError_t launch_dma(int tile, const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale,
                      const float* w_scale_up, int64_t M, int64_t K, int64_t N, int32_t* acc, void* out,
                      hipStream_t s) {
  if (tile == 256) return launch_dma_cfg<ABITS, 256, 256, 2, 4, MODE, 3>(codes, deq, Wq, w_scale, w_scale_up, M, K, N,
                                                                         acc, out, s);
  // 64 x 128 tiles of four waves (32 x 64 each), four stage buffers (loads three stages ahead:
  // these problems have few stages, so the first loads' latency weighs), 64 KB (INT8: 48 KB) of
  // LDS and 136 registers: two (INT8: three) blocks share a CU, so problems of a few hundred
  // tiles still put two waves on every SIMD
  if (tile == 64) return launch_dma_cfg<ABITS, 64, 128, 2, 2, MODE, 4>(codes, deq, Wq, w_scale, w_scale_up, M, K, N,
                                                                      acc, out, s);
  return launch_dma_cfg<ABITS, 128, 256, 1, 4, MODE, 2>(codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
}

}  // namespace

bool gemm_dma_ok(int64_t K, int abits) { return K % (abits == 4 ? 256 : 128) == 0 && K >= 256; }

hipError_t launch_gemm_dma(int tile, int mode, const uint8_t* codes, const float* deq, const uint8_t* Wq,
                           const float* w_scale, const float* w_scale_up, int64_t M, int64_t K, int64_t N, int abits,
                           int32_t* acc, void* out, hipStream_t s) {
  if (abits == 4) {
    switch (mode) {
      case 0: return launch_dma<4, 0>(tile, codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
      case 1: return launch_dma<4, 1>(tile, codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
      case 2: return launch_dma<4, 2>(tile, codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
      default: return launch_dma<4, 3>(tile, codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
    }
  }
  switch (mode) {
    case 0: return launch_dma<8, 0>(tile, codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
    case 1: return launch_dma<8, 1>(tile, codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
    case 2: return launch_dma<8, 2>(tile, codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
    default: return launch_dma<8, 3>(tile, codes, deq, Wq, w_scale, w_scale_up, M, K, N, acc, out, s);
  }
}

}  // namespace hbl
