/*
 * hbl_oracle.c — CPU oracle of the H-BitLinear forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this file's library.  The product path (the HIP kernels
 * and their C ABI) shares no code, header, table or helper with it.
 *
 * Plain, slow, scalar C11.  OpenMP is used only to run independent token rows (or
 * independent weight rows) on several cores; every floating-point operation inside a
 * row happens in the order written here.  Build with -O2 -ffp-contract=off and without
 * fast-math so that every float expression rounds as written (no FMA contraction).
 *
 * Sources (the scraped pages drop every equation; what each step follows is named at the
 * step):
 *  [V2]  "BitNet v2: Native 4-bit Activations with Hadamard Transformation for 1-bit LLMs",
 *        arXiv abstract page, and the Traditional-Chinese write-up of the paper,
 *        sections "BitNet v2：原生4位激活" and "H-BitLinear模塊".
 *  [CPP] the bitnet.cpp news article, section "6 页论文，引入 1 bit LLM" (absmean weight
 *        rounding to {-1,0,1}; activations scaled into [-Qb, Qb] without a zero point;
 *        RMSNorm, SwiGLU, no biases).
 *
 * Precision.  The pages fix no precision.  Every step that decides an integer (ternary
 * weight, activation code) is taken in fp32, the precision of the GPU kernels, so both
 * sides make the same decision; sums that only feed a scale (alpha, the RMS) are taken in
 * fp64.  orc_fwht_f64 and orc_dense_reference give an fp64 reference that the tests use to
 * bound the fp32 path's deviation.
 *
 * Parity pins: every function here is pinned by a CPU test against something other than
 * itself (Sylvester/SciPy Hadamard matrices, closed forms, hand-computed fixtures, integer
 * matmul, the quantisation error bound).  See the test files named test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

static float bf16_bits_to_f32(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16; /* a bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static float load_x(const void* x, int dtype, int64_t idx) {
  if (dtype == ORC_BF16) return bf16_bits_to_f32(((const uint16_t*)x)[idx]);
  return ((const float*)x)[idx];
}

/* ------------------------------------------------------------------------------------
 * Hadamard transform [V2, section H-BitLinear模塊: online Hadamard transform computed by
 * the fast Hadamard transform in O(n log n); a Hadamard matrix has +-1 entries and
 * mutually orthogonal rows].
 *
 * Textbook in-place butterfly: for h = 1, 2, 4, ..., n/2 and every pair (j, j+h) inside a
 * block of 2h, (a, b) -> (a+b, a-b).  The result is H_n v for the Sylvester matrix
 * H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]], i.e. H_n[i][j] = (-1)^popcount(i & j).
 * Unnormalised; n must be a power of two.
 * ------------------------------------------------------------------------------------ */
void orc_fwht_f32(float* v, int64_t n) {
  for (int64_t h = 1; h < n; h *= 2)
    for (int64_t i = 0; i < n; i += 2 * h)
      for (int64_t j = i; j < i + h; ++j) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

void orc_fwht_f64(double* v, int64_t n) {
  for (int64_t h = 1; h < n; h *= 2)
    for (int64_t i = 0; i < n; i += 2 * h)
      for (int64_t j = i; j < i + h; ++j) {
        double a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

/* ------------------------------------------------------------------------------------
 * Weight ternarisation [V2, section H-BitLinear模塊: per-tensor absmean quantisation of
 * the weights to {-1, 0, 1}; CPP: scale the matrix by its mean absolute value, then round
 * each entry to the nearest of -1, 0, 1].
 *   S = sum_n ( sum_k |W[n,k]| ), both ascending, in fp64 (row sums first)
 *   alpha = max((float)(S / (N*K)), 1e-5f)
 *   t = clamp(rint(fl32(W / alpha)), -1, 1)        rint: round half to even
 * T is N*K int8 (row-major).  Returns 0, or -1 on a bad argument.
 * ------------------------------------------------------------------------------------ */
int orc_quantize_weights(const float* W, int64_t N, int64_t K, int8_t* T, float* alpha_out) {
  if (!W || !T || !alpha_out || N <= 0 || K <= 0) return -1;
  double* row_sum = (double*)malloc((size_t)N * sizeof(double));
  if (!row_sum) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += fabs((double)W[n * K + k]);
    row_sum[n] = s;
  }
  double S = 0.0;
  for (int64_t n = 0; n < N; ++n) S += row_sum[n];
  free(row_sum);
  float alpha = (float)(S / ((double)N * (double)K));
  if (!(alpha >= 1e-5f)) alpha = 1e-5f;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      float r = rintf(W[n * K + k] / alpha);
      if (r > 1.0f) r = 1.0f;
      if (r < -1.0f) r = -1.0f;
      T[n * K + k] = (int8_t)r;
    }
  *alpha_out = alpha;
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Activation quantisation of one row [V2, section H-BitLinear模塊: LN, then the online
 * Hadamard transform, then per-token INT8 / INT4 quantisation; CPP: activations scaled
 * into [-Qb, Qb] without a zero point].  Per-token absmax with Qb = 2^(abits-1) - 1.
 *
 *   xf = (float)x;  u = norm ? fl32(xf * gamma) : xf
 *   r  = norm ? (float)(1 / sqrt(sum(xf^2 in fp64)/K + eps)) : 1
 *   z  = use_h ? FWHT_fp32(u) : u
 *   g  = max |z|; g < 2^-120 (this covers g == 0) -> q = 0, deq = 0, so that Qb/g
 *        below stays finite
 *   s  = fl32(Qb / g);  q = clamp(rint(fl32(z * s)), -Qb-1, Qb)
 *   deq = fl32(fl32(fl32(g / Qb) * r) * hK),  hK = use_h ? (float)(1/sqrt(K)) : 1
 *
 * The normalisation factors r and 1/sqrt(K) are applied to deq instead of to u and z:
 * absmax codes do not change under a positive per-row scale, so this is the same
 * quantiser, and the codes do not depend on how the RMS sum is ordered.
 * q: M*K int8 (unpacked), deq: M floats, rnorm (may be NULL): M floats of r.
 * ------------------------------------------------------------------------------------ */
int orc_quantize_activations_stat(const void* x, int dtype, int64_t M, int64_t K, int norm,
                                  const float* gamma, float eps, int abits, int use_h, int stat, int8_t* q,
                                  float* deq, float* rnorm) {
  if (M < 0 || K <= 0 || (abits != 4 && abits != 8) || (stat != 0 && stat != 1)) return -1;
  if (M > 0 && (!x || !q || !deq)) return -1;
  if (use_h && (K & (K - 1)) != 0) return -1;
  const int Qb = (abits == 4) ? 7 : 127;
  const float hK = use_h ? (float)(1.0 / sqrt((double)K)) : 1.0f;
  int bad = 0;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    float* z = (float*)malloc((size_t)K * sizeof(float));
    if (!z) {
      bad = 1;
      continue;
    }
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      float xf = load_x(x, dtype, m * K + k);
      if (norm) {
        ss += (double)xf * (double)xf;
        z[k] = gamma ? xf * gamma[k] : xf;
      } else {
        z[k] = xf;
      }
    }
    float r = 1.0f;
    if (norm) r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    if (rnorm) rnorm[m] = r;
    if (use_h) orc_fwht_f32(z, K);
    if (stat == 1) {
      /* absmean statistic: the pages' absmean function (scale by the mean absolute value,
       * round to the nearest integer, clip to the code range) applied to the INT4/INT8 grid:
       * b = (float)(sum_k |z_k| in fp64, ascending / K); s = fl32(1 / b);
       * q = clamp(rint_ne(fl32(z * s)), -Qb-1, Qb); deq = fl32(fl32(b * r) * hK). */
      double sa = 0.0;
      for (int64_t k = 0; k < K; ++k) sa += (double)fabsf(z[k]);
      const float b = (float)(sa / (double)K);
      if (b < 0x1p-120f) {
        for (int64_t k = 0; k < K; ++k) q[m * K + k] = 0;
        deq[m] = 0.0f;
      } else {
        const float s = 1.0f / b;
        for (int64_t k = 0; k < K; ++k) {
          float v = rintf(z[k] * s);
          if (v > (float)Qb) v = (float)Qb;
          if (v < (float)(-Qb - 1)) v = (float)(-Qb - 1);
          q[m * K + k] = (int8_t)v;
        }
        float d = b * r;
        d = d * hK;
        deq[m] = d;
      }
      free(z);
      continue;
    }
    float g = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      float a = fabsf(z[k]);
      if (a > g) g = a;
    }
    if (g < 0x1p-120f) {
      for (int64_t k = 0; k < K; ++k) q[m * K + k] = 0;
      deq[m] = 0.0f;
    } else {
      float s = (float)Qb / g;
      for (int64_t k = 0; k < K; ++k) {
        float v = rintf(z[k] * s);
        if (v > (float)Qb) v = (float)Qb;
        if (v < (float)(-Qb - 1)) v = (float)(-Qb - 1);
        q[m * K + k] = (int8_t)v;
      }
      float d = g / (float)Qb;
      d = d * r;
      d = d * hK;
      deq[m] = d;
    }
    free(z);
  }
  return bad ? -1 : 0;
}

int orc_quantize_activations(const void* x, int dtype, int64_t M, int64_t K, int norm,
                             const float* gamma, float eps, int abits, int use_h, int8_t* q, float* deq,
                             float* rnorm) {
  return orc_quantize_activations_stat(x, dtype, M, K, norm, gamma, eps, abits, use_h, 0, q, deq, rnorm);
}

/* ------------------------------------------------------------------------------------
 * Integer GEMM: acc[m,n] = sum_k q[m,k] * t[n,k] (exact in int32 for |q| <= 128,
 * |t| <= 1, K <= 2^24) [V2, section H-BitLinear模塊: the quantised matmul;
 * CPP: with ternary weights the product needs only additions].
 * ------------------------------------------------------------------------------------ */
int orc_gemm_s32(const int8_t* q, const int8_t* T, int64_t M, int64_t K, int64_t N, int32_t* acc) {
  if (M < 0 || K <= 0 || N <= 0) return -1;
  if (M > 0 && (!q || !T || !acc)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      int32_t s = 0;
      for (int64_t k = 0; k < K; ++k) s += (int32_t)q[m * K + k] * (int32_t)T[n * K + k];
      acc[m * N + n] = s;
    }
  return 0;
}

/* Dequantisation epilogue: y = fl32(fl32((float)acc * deq[m]) * alpha). */
int orc_dequant(const int32_t* acc, const float* deq, float alpha, int64_t M, int64_t N, float* y) {
  if (M < 0 || N <= 0) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      float v = (float)acc[m * N + n] * deq[m];
      y[m * N + n] = v * alpha;
    }
  return 0;
}

/* The whole forward on M rows: quantise activations, integer GEMM, dequantise.
 * T (N*K int8) and alpha come from orc_quantize_weights.  q_out/acc_out/deq_out may be
 * NULL; when given they receive the intermediate results (M*K, M*N, M). */
int orc_forward_stat(const void* x, int dtype, const int8_t* T, float alpha, int64_t M, int64_t K, int64_t N,
                     int abits, int use_h, int norm, const float* gamma, float eps, int stat, float* y,
                     int8_t* q_out, int32_t* acc_out, float* deq_out) {
  if (M < 0 || K <= 0 || N <= 0) return -1;
  if (M == 0) return 0;
  int8_t* q = q_out ? q_out : (int8_t*)malloc((size_t)(M * K));
  int32_t* acc = acc_out ? acc_out : (int32_t*)malloc((size_t)(M * N) * sizeof(int32_t));
  float* deq = deq_out ? deq_out : (float*)malloc((size_t)M * sizeof(float));
  int rc = -1;
  if (q && acc && deq) {
    rc = orc_quantize_activations_stat(x, dtype, M, K, norm, gamma, eps, abits, use_h, stat, q, deq, NULL);
    if (rc == 0) rc = orc_gemm_s32(q, T, M, K, N, acc);
    if (rc == 0) rc = orc_dequant(acc, deq, alpha, M, N, y);
  }
  if (!q_out) free(q);
  if (!acc_out) free(acc);
  if (!deq_out) free(deq);
  return rc;
}

int orc_forward(const void* x, int dtype, const int8_t* T, float alpha, int64_t M, int64_t K, int64_t N,
                int abits, int use_h, int norm, const float* gamma, float eps, float* y, int8_t* q_out,
                int32_t* acc_out, float* deq_out) {
  return orc_forward_stat(x, dtype, T, alpha, M, K, N, abits, use_h, norm, gamma, eps, 0, y, q_out, acc_out,
                          deq_out);
}

/* SwiGLU gate of the FFN [V2, section BitNet v2：原生4位激活: RMS normalisation, SwishGLU,
 * no bias; CPP: RMSNorm, SwiGLU]: h = silu(g) * u with silu(v) = v / (1 + e^-v), computed
 * in fp64 and rounded once to fp32. */
void orc_swiglu(const float* g, const float* u, int64_t n, float* h) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double gv = (double)g[i];
    double s = gv / (1.0 + exp(-gv));
    h[i] = (float)(s * (double)u[i]);
  }
}

/* fp32 -> bfloat16, round to nearest with ties to even.  bfloat16 keeps the sign, the
 * 8-bit exponent and the top 7 fraction bits of binary32, so it has 8 significant bits and
 * the same exponent range: a value of magnitude in [2^e, 2^(e+1)) is rounded to a multiple
 * of 2^(e-7), and values below 2^-126 to multiples of 2^-133 (the subnormal spacing).  The
 * rounded value is exact in binary32; its top 16 bits are the bfloat16 pattern.  Results of
 * magnitude 2^128 or more overflow to infinity. */
void orc_round_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    const float f = in[i];
    float r;
    if (isnan(f)) {
      out[i] = (uint16_t)(signbit(f) ? 0xFFC0u : 0x7FC0u);
      continue;
    } else if (isinf(f) || f == 0.0f) {
      r = f;
    } else {
      int e;
      frexp((double)f, &e); /* |f| in [2^(e-1), 2^e) */
      int qexp = (e - 1) - 7;
      if (qexp < -133) qexp = -133;
      const double q = ldexp(1.0, qexp);
      const double v = rint((double)f / q) * q; /* exact scaling, one rounding (ties to even) */
      r = fabs(v) >= 0x1p128 ? (v > 0 ? INFINITY : -INFINITY) : (float)v;
    }
    uint32_t bits;
    memcpy(&bits, &r, sizeof bits);
    out[i] = (uint16_t)(bits >> 16);
  }
}

/* ------------------------------------------------------------------------------------
 * QKV state quantisation [V2, text of Tables 2 and 3 (low-bit attention): the Q, K and V
 * states are quantised after RoPE, each head directly to unsigned integers with the absmax
 * function and no calibration data; a 3-bit KV cache keeps the accuracy of a full-precision
 * one].  Reading: a head vector x of length d is mapped linearly from [-g, g], g = max|x|,
 * onto the unsigned grid 0 .. L with L = 2^bits - 1 (both ends reachable):
 *     s = fl32(L / fl32(2g)),   c = L/2 (exact),
 *     u = clamp(rint_ne(fl32(fl32(x*s) + c)), 0, L)
 * and g < 2^-120 takes s = 0, so a zero head gives u = rint_ne(c) everywhere.
 * Reconstruction: xhat = fl32(fl32(u - c) * D) with D = fl32(fl32(2g) / L).
 * u: rows*d unpacked codes (uint8); gamma: one g per head row.
 * ------------------------------------------------------------------------------------ */
int orc_quantize_qkv(const void* x, int dtype, int64_t rows, int64_t d, int bits, uint8_t* u, float* gamma) {
  if (rows < 0 || d <= 0 || bits < 2 || bits > 8) return -1;
  if (rows > 0 && (!x || !u || !gamma)) return -1;
  const float L = (float)((1 << bits) - 1);
  const float c = L / 2.0f;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float g = 0.0f;
    for (int64_t i = 0; i < d; ++i) {
      float a = fabsf(load_x(x, dtype, r * d + i));
      if (a > g) g = a;
    }
    gamma[r] = g;
    const float s = g < 0x1p-120f ? 0.0f : L / (2.0f * g);
    for (int64_t i = 0; i < d; ++i) {
      float v = load_x(x, dtype, r * d + i) * s;
      v = rintf(v + c);
      if (v < 0.0f) v = 0.0f;
      if (v > L) v = L;
      u[r * d + i] = (uint8_t)v;
    }
  }
  return 0;
}

int orc_dequantize_qkv(const uint8_t* u, const float* gamma, int64_t rows, int64_t d, int bits, float* out) {
  if (rows < 0 || d <= 0 || bits < 2 || bits > 8) return -1;
  const float L = (float)((1 << bits) - 1);
  const float c = L / 2.0f;
  for (int64_t r = 0; r < rows; ++r) {
    const float D = (2.0f * gamma[r]) / L;
    for (int64_t i = 0; i < d; ++i) out[r * d + i] = ((float)u[r * d + i] - c) * D;
  }
  return 0;
}

/* b-bit codes, least significant bit first: code i of a row occupies bits [b*i, b*i + b) of
 * the row's little-endian bit string; rows of d*b/8 bytes (d*b % 8 == 0). */
int orc_pack_bits(const uint8_t* u, int64_t rows, int64_t d, int bits, uint8_t* out) {
  if (rows < 0 || d <= 0 || bits < 1 || bits > 8 || (d * bits) % 8 != 0) return -1;
  const int64_t rb = d * bits / 8;
  memset(out, 0, (size_t)(rows * rb));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < d; ++i) {
      const unsigned v = u[r * d + i];
      if (v >> bits) return -1;
      for (int b = 0; b < bits; ++b) {
        const int64_t bit = i * bits + b;
        if ((v >> b) & 1u) out[r * rb + bit / 8] |= (uint8_t)(1u << (bit % 8));
      }
    }
  return 0;
}

int orc_unpack_bits(const uint8_t* in, int64_t rows, int64_t d, int bits, uint8_t* u) {
  if (rows < 0 || d <= 0 || bits < 1 || bits > 8 || (d * bits) % 8 != 0) return -1;
  const int64_t rb = d * bits / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < d; ++i) {
      unsigned v = 0;
      for (int b = 0; b < bits; ++b) {
        const int64_t bit = i * bits + b;
        v |= (unsigned)((in[r * rb + bit / 8] >> (bit % 8)) & 1u) << b;
      }
      u[r * d + i] = (uint8_t)v;
    }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Packed formats (the header of the C ABI documents them; not given by the pages).
 * ------------------------------------------------------------------------------------ */

/* Wq: N rows of K/4 bytes; 32-bit little-endian words of 16 weights; weight c of a word
 * (k = 16w + c) in the 2-bit field p = 4*(c%4) + c/4; two's complement 2-bit codes. */
int orc_pack_weights(const int8_t* T, int64_t N, int64_t K, uint8_t* Wq) {
  if (N <= 0 || K <= 0 || (K % 16) != 0) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t w = 0; w < K / 16; ++w) {
      uint32_t word = 0;
      for (int c = 0; c < 16; ++c) {
        int t = T[n * K + 16 * w + c];
        uint32_t field = (uint32_t)t & 3u; /* -1 -> 0b11, 0 -> 0b00, 1 -> 0b01 */
        int p = 4 * (c % 4) + c / 4;
        word |= field << (2 * p);
      }
      uint8_t* dst = Wq + n * (K / 4) + 4 * w;
      dst[0] = (uint8_t)(word & 0xff);
      dst[1] = (uint8_t)((word >> 8) & 0xff);
      dst[2] = (uint8_t)((word >> 16) & 0xff);
      dst[3] = (uint8_t)((word >> 24) & 0xff);
    }
  return 0;
}

int orc_unpack_weights(const uint8_t* Wq, int64_t N, int64_t K, int8_t* T) {
  if (N <= 0 || K <= 0 || (K % 16) != 0) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t w = 0; w < K / 16; ++w) {
      const uint8_t* src = Wq + n * (K / 4) + 4 * w;
      uint32_t word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16) |
                      ((uint32_t)src[3] << 24);
      for (int c = 0; c < 16; ++c) {
        int p = 4 * (c % 4) + c / 4;
        uint32_t field = (word >> (2 * p)) & 3u;
        T[n * K + 16 * w + c] = (int8_t)(field == 3u ? -1 : (int)field); /* 0b10 is invalid */
      }
    }
  return 0;
}

/* codes: abits 8 -> the int8 values in order; abits 4 -> 8-byte groups of 16 codes, byte
 * j holding code (j%4) + 8*(j/4) in the low nibble and that code + 4 in the high nibble. */
int orc_pack_codes(const int8_t* q, int64_t M, int64_t K, int abits, uint8_t* codes) {
  if (M < 0 || K <= 0) return -1;
  if (abits == 8) {
    for (int64_t i = 0; i < M * K; ++i) codes[i] = (uint8_t)q[i];
    return 0;
  }
  if (abits != 4 || (K % 16) != 0) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t G = 0; G < K / 16; ++G)
      for (int j = 0; j < 8; ++j) {
        int c0 = (j % 4) + 8 * (j / 4);
        uint8_t lo = (uint8_t)q[m * K + 16 * G + c0] & 0x0f;
        uint8_t hi = (uint8_t)q[m * K + 16 * G + c0 + 4] & 0x0f;
        codes[m * (K / 2) + 8 * G + j] = (uint8_t)(lo | (hi << 4));
      }
  return 0;
}

int orc_unpack_codes(const uint8_t* codes, int64_t M, int64_t K, int abits, int8_t* q) {
  if (M < 0 || K <= 0) return -1;
  if (abits == 8) {
    for (int64_t i = 0; i < M * K; ++i) q[i] = (int8_t)codes[i];
    return 0;
  }
  if (abits != 4 || (K % 16) != 0) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t G = 0; G < K / 16; ++G)
      for (int j = 0; j < 8; ++j) {
        int c0 = (j % 4) + 8 * (j / 4);
        uint8_t b = codes[m * (K / 2) + 8 * G + j];
        int lo = b & 0x0f, hi = (b >> 4) & 0x0f;
        q[m * K + 16 * G + c0] = (int8_t)(lo >= 8 ? lo - 16 : lo);
        q[m * K + 16 * G + c0 + 4] = (int8_t)(hi >= 8 ? hi - 16 : hi);
      }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * FP6 / FP4 storage of the same codes (the C ABI header documents the layouts).  The
 * encodings follow the OCP microscaling element formats: FP6 E2M3 is sign | 2-bit
 * exponent (bias 1) | 3-bit mantissa, value (-1)^s * 2^(e-1) * (1 + m/8) for e > 0 and
 * (-1)^s * m/8 for e = 0; FP4 E2M1 is sign | 2-bit exponent (bias 1) | 1-bit mantissa.
 * Only integers are encoded here (INT4 codes |q| <= 7, ternary weights), all exactly.
 * ------------------------------------------------------------------------------------ */
static unsigned fp6_e2m3_of_int(int q) {
  unsigned sign = q < 0 ? 1u : 0u;
  unsigned a = (unsigned)(q < 0 ? -q : q);
  unsigned code;
  if (a == 0) {
    code = 0;
  } else {
    unsigned e = 0; /* floor(log2 a) */
    while ((a >> (e + 1)) != 0) ++e;
    /* a = 2^e * (1 + m/8)  =>  m = (a - 2^e) * 8 / 2^e, exact for a <= 7 */
    unsigned m = ((a - (1u << e)) * 8u) >> e;
    code = ((e + 1u) << 3) | m;
  }
  return (sign << 5) | code;
}

static int int_of_fp6_e2m3(unsigned code) {
  unsigned e = (code >> 3) & 3u, m = code & 7u;
  double v = e == 0 ? m / 8.0 : ldexp(1.0 + m / 8.0, (int)e - 1);
  if (code & 0x20u) v = -v;
  return (int)v;
}

int orc_pack_codes_fp6(const int8_t* q, int64_t M, int64_t K, uint8_t* out) {
  if (M < 0 || K <= 0 || (K % 4) != 0) return -1;
  const int64_t rb = K / 4 * 3;
  for (int64_t m = 0; m < M; ++m) {
    uint8_t* row = out + m * rb;
    for (int64_t b = 0; b < rb; ++b) row[b] = 0;
    for (int64_t k = 0; k < K; ++k) {
      int qv = q[m * K + k];
      if (qv < -7 || qv > 7) return -1;
      unsigned c = fp6_e2m3_of_int(qv);
      int64_t bit = 6 * k;
      for (int i = 0; i < 6; ++i)
        if ((c >> i) & 1u) row[(bit + i) / 8] |= (uint8_t)(1u << ((bit + i) % 8));
    }
  }
  return 0;
}

int orc_unpack_codes_fp6(const uint8_t* codes, int64_t M, int64_t K, int8_t* q) {
  if (M < 0 || K <= 0 || (K % 4) != 0) return -1;
  const int64_t rb = K / 4 * 3;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) {
      unsigned c = 0;
      int64_t bit = 6 * k;
      for (int i = 0; i < 6; ++i) c |= (unsigned)((codes[m * rb + (bit + i) / 8] >> ((bit + i) % 8)) & 1u) << i;
      q[m * K + k] = (int8_t)int_of_fp6_e2m3(c);
    }
  return 0;
}

int orc_pack_weights_fp4(const int8_t* T, int64_t N, int64_t K, uint8_t* out) {
  if (N <= 0 || K <= 0 || (K % 2) != 0) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; k += 2) {
      unsigned nib[2];
      for (int i = 0; i < 2; ++i) {
        int t = T[n * K + k + i];
        /* E2M1: 1.0 = exponent 1 (bias 1), mantissa 0 -> 0b0010; sign is bit 3 */
        nib[i] = t == 0 ? 0u : ((t < 0 ? 8u : 0u) | 2u);
      }
      out[n * (K / 2) + k / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
    }
  return 0;
}
