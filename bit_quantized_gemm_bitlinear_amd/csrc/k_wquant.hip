// k_wquant.hip — per-tensor absmean ternarisation of a weight matrix and 2-bit packing.
//
// BitNet v2 write-up, section H-BitLinear模塊: the weights are ternarised to {-1, 0, 1}
// with a per-tensor absmean scale; bitnet.cpp article, section "6 页论文，引入 1 bit LLM":
// divide the matrix by its mean absolute value and round to the nearest integer in
// {-1, 0, 1}.  The mean is summed in a fixed order (fp64, each row ascending in k, then
// the row sums ascending in n) so the scale is reproducible bit for bit.
//
// This runs once per weight matrix, outside the per-token path; it is three launches:
//   wq_rowsum   one lane per weight row, sequential fp64 sum of |W| over k
//   wq_scale    one lane: ordered sum of the row sums, alpha = max((float)(S/(N K)), 1e-5)
//   wq_pack     one thread per 16-weight word: t = clamp(rint(W/alpha), -1, 1), 2-bit fields
//
// The fixed order makes the scale a chain of K + N dependent fp64 additions, so both sums are
// latency-bound: what matters is that every lane of a chain finds its operands on chip, ready
// to add, when it needs them.  wq_rowsum has one wave stream and convert the rows for another
// that only adds; wq_scale stages the row sums through LDS and reads them 16 at a time.
#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

// Row sums.  A block owns RS_ROWS = 16 rows and has two waves.  The chain of each row (one
// fp64 addition per weight, in ascending k) runs in lanes 0..15 of the second wave, which does
// nothing else: its additions wait only for one another.  The first wave feeds it.  It streams
// the rows through a ring of NB float chunks (64 weights per row, 4 KB) in LDS with
// 16-byte-per-lane loads straight into LDS, issued NB chunks ahead (lanes 16 r' + p of load i
// fetch row 4 i + r', float4 p ^ row, so float4 j of row r sits at slot j ^ r), and converts
// each chunk to fp64 |w| into a ring of double chunks, ahead of the chain
// (double pair m of row r at 16-byte slot m ^ r: the chain lanes' reads of pair m of their
// rows hit 16 different bank groups).  (fp32 -> fp64 conversion issues at a quarter of the
// addition rate, so a wave doing both per element would be held up by the conversions.)  One
// barrier per CPB chunks (3 CPB double slots: the feeder works CPB + 1 to 2 CPB chunks ahead
// of the chain).  NB = 8 and CPB = 2 (80 KB, two blocks per CU) when every block is resident at
// once anyway; with many rows NB = 4 and CPB = 1 (40 KB) let four blocks share a CU.
constexpr int RS_ROWS = 16, RS_CH = 64;
constexpr int RS_CHUNK_BYTES = RS_ROWS * RS_CH * 4;    // 4096: one float chunk
constexpr int RS_DROW = RS_CH * 8;                     // bytes per row of a double chunk
constexpr int RS_DCHUNK = RS_ROWS * RS_DROW;           // 8192

template <int NB, int CPB>
__global__ __launch_bounds__(128) void wq_rowsum(const float* __restrict__ W, int64_t N, int64_t K,
                                                 double* __restrict__ rowsum) {
  constexpr int DB = 3 * CPB;   // double slots
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NB * RS_CHUNK_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t dring[DB * RS_DCHUNK];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * RS_ROWS;
  const int rows = (int)min((int64_t)RS_ROWS, N - n0);
  const int C = (int)(K / RS_CH);   // chunks (K % 64 == 0)
  const int P = (C + CPB - 1) / CPB;   // barrier intervals: chunks CPB p .. CPB p + CPB - 1

  if (wave == 0) {
    // ---- feeder ----
    const int64_t rbytes = K * 4;
    const v4u_t rsrc = buffer_rsrc(W + n0 * K, (uint32_t)(rows * rbytes));
    uint32_t voff[4];   // rows past N re-read the last row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * i + (lane >> 4);
      voff[i] = (uint32_t)(min(r, rows - 1) * rbytes + 16 * ((lane & 15) ^ r));
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)ring;
    // chunk c (past the last chunk: the last one again) into float slot c % NB
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
      const uint32_t base = lds0 + (uint32_t)((c % NB) * RS_CHUNK_BYTES);
      const uint32_t soff = (uint32_t)min(c, C - 1) * (RS_CH * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(rsrc, voff[i], soff, base + 1024 * i);
    };
    // Float chunk c -> double chunk c: lane 4 r + q converts weights 16 q .. 16 q + 15 of row r.
    // Then chunk c + NB is loaded into the float slot just read.  Every call issues the same
    // four loads, so chunk c is complete once the NB - 1 younger chunks' loads are pending.
    const int r = lane >> 2, q = lane & 3;
    auto convert = [&](int c) __attribute__((always_inline)) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (NB - 1)) : "memory");
      const uint8_t* src = ring + (c % NB) * RS_CHUNK_BYTES + r * (RS_CH * 4);
      float4 f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = *reinterpret_cast<const float4*>(src + 16 * ((4 * q + i) ^ r));
      uint8_t* dst = dring + (c % DB) * RS_DCHUNK + r * RS_DROW;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 8 * q + 2 * i;   // double pairs m, m + 1 of the row
        *reinterpret_cast<double2*>(dst + 16 * (m ^ r)) = double2{(double)fabsf(f[i].x), (double)fabsf(f[i].y)};
        *reinterpret_cast<double2*>(dst + 16 * ((m + 1) ^ r)) = double2{(double)fabsf(f[i].z), (double)fabsf(f[i].w)};
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the float slot has been read
      load_chunk(c + NB);
    };
#pragma unroll
    for (int c = 0; c < NB; ++c) load_chunk(c);
    // chunks 0 .. CPB before the first barrier; in interval p, chunks CPB p + CPB + 1 ..
    // CPB p + 2 CPB, whose slots held chunks of interval p - 2 and the first of p - 1
    for (int c = 0; c <= CPB; ++c)
      if (c < C) convert(c);
    __syncthreads();
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int k = 1; k <= CPB; ++k)
        if (CPB * p + CPB + k < C) convert(CPB * p + CPB + k);
      __syncthreads();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still write LDS at exit
  } else {
    // ---- chain ----  Double chunk c is complete from the barrier after its conversion on;
    // its slot is rewritten only after the barrier that follows the last addition from it.
    // The reads run one group of 16 weights ahead of the additions, across chunk boundaries.
    // The loop is unrolled over the DB slots, so a read is a per-lane offset (computed once)
    // plus a constant: the chain's wave issues nothing but reads, waits and additions.
    const int r = lane & 15;
    constexpr int G = 16, NG = RS_CH / G;   // weights per group, groups per chunk
    uint32_t off[RS_CH / 2];                // double pair j of this lane's row, in a slot
#pragma unroll
    for (int j = 0; j < RS_CH / 2; ++j) off[j] = (uint32_t)(r * RS_DROW + 16 * (j ^ r));
    auto read_group = [&](int slot, int g, double (&d)[G]) __attribute__((always_inline)) {
      const uint8_t* src = dring + slot * RS_DCHUNK;
#pragma unroll
      for (int i = 0; i < G / 2; ++i) {
        const double2 v = *reinterpret_cast<const double2*>(src + off[G / 2 * g + i]);
        d[2 * i] = v.x;
        d[2 * i + 1] = v.y;
      }
    };
    double s = 0.0;
    double ga[G], gb[G];
    // the additions of the chunk in slot `slot`
    auto chunk = [&](int slot) __attribute__((always_inline)) {
      if (lane < RS_ROWS) {
#pragma unroll
        for (int g = 0; g < NG; g += 2) {
          // (each empty statement keeps the additions after the reads issued before it)
          read_group(slot, g + 1, gb);
          asm volatile("" : "+v"(s)::"memory");
#pragma unroll
          for (int u = 0; u < G; ++u) s += ga[u];
          // the last group's successor is group 0 of the next chunk (past the last chunk: a
          // stale slot, never added)
          if (g + 2 < NG) read_group(slot, g + 2, ga);
          else read_group((slot + 1) % DB, 0, ga);
          asm volatile("" : "+v"(s)::"memory");
#pragma unroll
          for (int u = 0; u < G; ++u) s += gb[u];
        }
      }
    };
    // interval p, its first chunk in slot `slot0`, then the barrier after it (every addition
    // from its chunks is done, so their reads have returned)
    auto interval = [&](int p, int slot0) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < CPB; ++k)
        if (CPB * p + k < C) chunk(slot0 + k);
      asm volatile("" : "+v"(s)::"memory");
      __syncthreads();
    };
    __syncthreads();   // double chunks 0 .. CPB are ready
    if (lane < RS_ROWS) read_group(0, 0, ga);
    int p = 0;
    for (; p + 3 <= P; p += 3) {
      interval(p, 0);
      interval(p + 1, CPB);
      interval(p + 2, 2 * CPB);
    }
    if (p < P) interval(p, 0);
    if (p + 1 < P) interval(p + 1, CPB);
    if (lane < rows) rowsum[n0 + lane] = s;
  }
}

// Ordered sum of the row sums by lane 0 of one 256-thread block.  The row sums pass through
// LDS in chunks of SC_CH: while lane 0 adds chunk c, every thread has chunk c + 1 in flight
// into registers; lane 0 reads LDS 16 doubles ahead of its chain.
constexpr int SC_CH = 4096;

__global__ __launch_bounds__(256) void wq_scale(const double* __restrict__ rowsum, int64_t N, int64_t K,
                                                float* __restrict__ w_scale) {
  __shared__ double buf[2][SC_CH];
  const int tid = threadIdx.x;
  constexpr int PER = SC_CH / 256;   // doubles per thread per chunk
  const int64_t C = (N + SC_CH - 1) / SC_CH;
  double nxt[PER];
  auto fetch = [&](int64_t c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t n = c * SC_CH + i * 256 + tid;
      nxt[i] = n < N ? rowsum[n] : 0.0;
    }
  };
  auto put = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER; ++i) buf[b][i * 256 + tid] = nxt[i];
  };
  fetch(0);
  put(0);
  __syncthreads();
  double S = 0.0;
  for (int64_t c = 0; c < C; ++c) {
    if (c + 1 < C) fetch(c + 1);
    if (tid == 0) {
      const int cnt = (int)min((int64_t)SC_CH, N - c * SC_CH);
      const double* p = buf[c & 1];
      int i = 0;
      for (; i + 16 <= cnt; i += 16) {
        double v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = p[i + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) S += v[u];
      }
      for (; i < cnt; ++i) S += p[i];
    }
    if (c + 1 < C) put((c + 1) & 1);
    __syncthreads();
  }
  if (tid == 0) {
    float alpha = (float)(S / ((double)N * (double)K));
    if (!(alpha >= 1e-5f)) alpha = 1e-5f;
    w_scale[0] = alpha;
  }
}

// Field position of weight c (0..15) inside its 32-bit word: p = 4*(c%4) + c/4.  With this
// order, shifting the word left by 6, 4, 2, 0 and masking 0xC0C0C0C0 yields four int8
// registers whose byte b holds 64*t for weights c = 4j + b, j = 0..3, in natural order.
__global__ __launch_bounds__(256) void wq_pack(const float* __restrict__ W, int64_t words,
                                               const float* __restrict__ w_scale, uint32_t* __restrict__ Wq) {
  const float alpha = w_scale[0];
  for (int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x; w < words; w += (int64_t)gridDim.x * 256) {
    const float4* p = reinterpret_cast<const float4*>(W + 16 * w);
    float e[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 f = p[i];
      e[4 * i + 0] = f.x;
      e[4 * i + 1] = f.y;
      e[4 * i + 2] = f.z;
      e[4 * i + 3] = f.w;
    }
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      float r = __builtin_rintf(e[c] / alpha);
      r = fminf(fmaxf(r, -1.0f), 1.0f);
      uint32_t field = (uint32_t)(int)r & 3u;
      word |= field << (2 * (4 * (c & 3) + (c >> 2)));
    }
    Wq[w] = word;
  }
}

}  // namespace

hipError_t launch_wquant(const float* W, int64_t N, int64_t K, uint8_t* Wq, float* w_scale, double* ws,
                         hipStream_t s) {
  const int64_t rblocks = (N + RS_ROWS - 1) / RS_ROWS;
  if (rblocks > 2 * CUS)
    hipLaunchKernelGGL((wq_rowsum<4, 1>), dim3((unsigned)rblocks), dim3(128), 0, s, W, N, K, ws);
  else
    hipLaunchKernelGGL((wq_rowsum<8, 2>), dim3((unsigned)rblocks), dim3(128), 0, s, W, N, K, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wq_scale, dim3(1), dim3(256), 0, s, ws, N, K, w_scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t words = N * K / 16;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(wq_pack, dim3((unsigned)blocks), dim3(256), 0, s, W, words, w_scale,
                     reinterpret_cast<uint32_t*>(Wq));
  return hipGetLastError();
}

}  // namespace hbl
