/*
 * hbl.h — C ABI of the H-BitLinear forward pass on AMD Instinct MI355X (gfx950).
 *
 * The layer (BitNet v2, "H-BitLinear" as described on the arXiv abstract page of
 * "BitNet v2: Native 4-bit Activations with Hadamard Transformation for 1-bit LLMs"
 * and in the section "H-BitLinear模塊" of the Traditional-Chinese write-up of that
 * paper) replaces the bias-free nn.Linear of the attention output projection Wo and
 * the FFN down projection Wdown.  For one token row x (length K) it computes
 *
 *     u  = RMSNorm(x)                      (optional; unit or given gamma)
 *     z  = H_K u                           (online fast Walsh-Hadamard transform)
 *     q  = absmax_quant(z) in INT4 or INT8 (per token, no zero point)
 *     y  = (q . t^T) * scales              (t = per-tensor absmean ternary weights)
 *
 * and the same without H for a plain BitLinear (all other linears of the model).
 *
 * Numerics (the pages drop every equation; the readings below are the contract, and
 * the test oracle implements exactly these steps on the CPU):
 *
 *  Weights (write-up, section H-BitLinear模塊: per-tensor absmean ternarisation;
 *  bitnet.cpp article, section "6 页论文，引入 1 bit LLM": scale by the mean absolute
 *  value, then round to the nearest of -1, 0, 1):
 *      S      = sum over rows n ascending of (sum over k ascending of |W[n,k]|), in fp64
 *      alpha  = max( (float)(S / (N*K)), 1e-5f )
 *      t[n,k] = clamp( rint_ne( fl32(W[n,k] / alpha) ), -1, 1 )
 *
 *  Activations, per row m (write-up, section H-BitLinear模塊: LN, then Hadamard by FHT,
 *  then INT8/INT4 quantisation; bitnet.cpp article: activations scaled into [-Qb, Qb]
 *  with no zero point).  Qb = 7 (abits 4) or 127 (abits 8):
 *      xf   = (float) x                                  (bf16 -> fp32 is exact)
 *      u_k  = norm ? fl32(xf_k * gamma_k) : xf_k           (gamma == NULL means gamma = 1)
 *      r    = norm ? (float)(1 / sqrt( (sum_k xf_k^2 in fp64, k ascending)/K + eps )) : 1
 *      z    = use_hadamard ? FWHT_fp32(u) : u             (butterfly stages h = 1,2,4,..,K/2,
 *                                                          each pair (j, j+h) -> (a+b, a-b) in fp32;
 *                                                          z = H_K u with H_K[i][j] = (-1)^popcount(i&j))
 *      g    = max_k |z_k|
 *      if g < 2^-120:  q = 0 and deq = 0          (covers g == 0; keeps Qb/g finite)
 *      else:       s = fl32(Qb / g);  q_k = clamp( rint_ne( fl32(z_k * s) ), -Qb-1, Qb )
 *                  deq = fl32( fl32( fl32(g / Qb) * r ) * hK ),  hK = use_hadamard ? (float)(1/sqrt(K)) : 1
 *  The Hadamard transform is the orthonormal one, H_K / sqrt(K); the 1/sqrt(K) and the
 *  RMSNorm factor r are folded into deq (absmax codes are invariant under any positive
 *  per-row scale, so the codes do not depend on them).
 *
 *  Summation order.  The steps above fix the result up to the order of fp32 sums.  bf16 rows
 *  with unit gamma and K = 2^10 .. 2^14 under the transform run five or six of its stages
 *  (index bits 0, 1, 2, 8, 9, and 10 when K >= 2^11) as products with H_32 on the bf16 matrix
 *  cores (exact products, fp32 sums in the matrix core's order) and the other stages in another
 *  order than above, and take r from an fp32 sum of squares (then fp64 across lanes) and
 *  v_rsq_f32.  z then agrees with the plain loop up to fp32 rounding: a code can move by one
 *  step when z*s lies within rounding of a half-integer (at most 1e-4 of the codes; a few per
 *  million on Gaussian rows), and deq by a few ulp.  On integer-valued rows whose transform stays below 2^24 in magnitude, with no norm,
 *  every sum is exact and codes and deq are exactly the above.  All other inputs (fp32 rows,
 *  a gamma, other K, no transform) follow the steps above exactly, with the RMS sum of squares
 *  in fp64 in another order (deq within 2 ulp).
 *
 *  GEMM and epilogue:
 *      acc[m,n] = sum_k q[m,k] * t[n,k]          (exact, int32)
 *      y[m,n]   = fl32( fl32( (float)acc[m,n] * deq[m] ) * alpha )
 *
 * Packed formats (not given by the pages; chosen so the GEMM can widen them to int8
 * MFMA operands with two or three bit operations per 32-bit word):
 *
 *  Wq — packed ternary weights, N rows of K/4 bytes, row-major.  Row n is a sequence of
 *       little-endian 32-bit words; word w holds the 16 weights k = 16w + c, c = 0..15.
 *       Weight c sits in the 2-bit field p = 4*(c % 4) + c/4 (bits 2p and 2p+1), encoded
 *       as 2-bit two's complement: 0b00 = 0, 0b01 = +1, 0b11 = -1 (0b10 never appears).
 *
 *  codes, abits = 8 — int8 two's complement, M rows of K bytes, natural order.
 *
 *  codes, abits = 4 — M rows of K/2 bytes.  Each 8-byte group G of a row holds the codes
 *       k = 16G + c, c = 0..15.  Byte j (0..7) of the group holds, as 4-bit two's
 *       complement nibbles, code c0 = (j % 4) + 8*(j / 4) in its low nibble and code c0+4
 *       in its high nibble.
 *
 *  deq — one fp32 per row.
 *
 *  FP6/FP4 variant of the a4 path (gfx950's scaled f8f6f4 matrix cores run FP6 x FP4 at
 *  twice the int8 rate; every INT4 code in [-7, 7] and every ternary weight is exact in
 *  these formats, so results are identical to the INT4/2-bit path):
 *  codes6 — the same INT4 absmax codes (Qb = 7), M rows of 3K/4 bytes; code k of a row sits
 *       at bits [6k, 6k+6) of the row read as a little-endian bit string, encoded as OCP FP6
 *       E2M3 (bit 5 sign, bits 4..3 exponent with bias 1, bits 2..0 mantissa): 0 -> 0x00,
 *       1 -> 0x08, 2 -> 0x10, 3 -> 0x14, 4 -> 0x18, 5 -> 0x1A, 6 -> 0x1C, 7 -> 0x1E, and
 *       -q -> 0x20 | code(q).
 *  Wq4  — ternary weights as OCP FP4 E2M1, N rows of K/2 bytes; weight k of a row in nibble
 *       k (low nibble first): 0 -> 0x0, +1 -> 0x2, -1 -> 0xA.
 *
 * Conventions for every entry point:
 *  - Every pointer argument is a device pointer (hipMalloc / torch CUDA memory) unless
 *    stated otherwise, 16-byte aligned.  The caller owns every buffer; the library never
 *    allocates device memory.  Its only mutable state is the static scratch array of
 *    hbl_forward_noalloc (one per GPU) and the pointers to it.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All work is
 *    enqueued asynchronously on that stream.  Calls on different streams are independent.
 *  - Arguments are validated synchronously, before any HIP call.  An invalid argument
 *    returns a status other than HBL_OK, enqueues nothing, and sets a per-thread message
 *    readable with hbl_last_error().  A kernel launch error returns HBL_ERR_HIP.  Faults
 *    inside kernels surface at the caller's next synchronisation of the stream.
 *  - Sizes are int64_t.  M == 0 is a valid no-op for every call that takes M.
 *  - Inputs with NaN or infinities give unspecified codes and outputs.
 *  - No C++ exception crosses this interface.
 */
#ifndef HBL_H_
#define HBL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HBL_OK = 0,
  HBL_ERR_INVALID_ARG = 1, /* null pointer, negative size, abits not 4/8, misaligned ... */
  HBL_ERR_UNSUPPORTED = 2, /* a valid request outside what the kernels implement       */
  HBL_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_bytes  */
  HBL_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed               */
} hbl_status;

typedef enum { HBL_F32 = 0, HBL_BF16 = 1 } hbl_dtype;
typedef enum { HBL_NORM_NONE = 0, HBL_NORM_RMS = 1 } hbl_norm;
/* Per-token activation statistic (see hbl_quantize_activations_stat). */
typedef enum { HBL_STAT_ABSMAX = 0, HBL_STAT_ABSMEAN = 1 } hbl_stat;

/* Limits of this implementation.
 *  K % 64 == 0 and 64 <= K <= HBL_MAX_K for every call.
 *  With use_hadamard, K is also a power of two and K <= HBL_MAX_K_HADAMARD
 *  (the transform keeps one fp32 row on chip).
 *  |acc| <= 127*K < 2^24 for K <= HBL_MAX_K, so (float)acc is exact. */
#define HBL_MAX_K 131072
#define HBL_MAX_K_HADAMARD 32768

/* Byte sizes of the packed buffers (0 for invalid arguments). */
size_t hbl_packed_weight_bytes(int64_t N, int64_t K);           /* N*K/4          */
size_t hbl_packed_act_bytes(int64_t M, int64_t K, int abits);   /* M*K*abits/8    */
/* Workspace of hbl_quantize_weights: N fp64 row sums.  */
size_t hbl_wquant_workspace_bytes(int64_t N, int64_t K);
/* Workspace of hbl_forward: the codes and deq of M rows (256-byte aligned pieces). */
size_t hbl_forward_workspace_bytes(int64_t M, int64_t K, int abits);

/* hbl_quantize_weights — per-tensor absmean ternarisation and 2-bit packing.
 * (write-up section H-BitLinear模塊; bitnet.cpp article section "6 页论文，引入 1 bit LLM")
 *  W        [N, K] fp32, row-major (out x in, the nn.Linear convention).
 *  Wq       [N, K/4] bytes, written in the Wq format above.
 *  w_scale  one fp32 on the device: alpha.
 *  ws       workspace of at least hbl_wquant_workspace_bytes(N, K) bytes.
 *  N >= 1.  Deterministic: alpha is computed in the fixed order stated above. */
hbl_status hbl_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* Wq, float* w_scale,
                                void* ws, size_t ws_bytes, void* stream);

/* hbl_quantize_activations — load, optional RMSNorm, optional online FWHT, per-token
 * absmax quantisation and packing (write-up section H-BitLinear模塊).
 *  x        [M, K] of dtype xt, row-major.
 *  gamma    [K] fp32 RMSNorm weight, or NULL for unit gamma; ignored if norm == NONE.
 *  norm_eps RMSNorm epsilon (finite, >= 0).
 *  codes    [M, K*abits/8] bytes in the codes format above.
 *  deq      [M] fp32 per-row dequantisation factor. */
hbl_status hbl_quantize_activations(const void* x, hbl_dtype xt, int64_t M, int64_t K, hbl_norm norm,
                                    const float* gamma, float norm_eps, int abits, int use_hadamard,
                                    uint8_t* codes, float* deq, void* stream);

/* GEMM kernels: M <= 64 token rows (the decode regime) run a kernel that streams every weight
 * byte once and splits K over the waves of a block; larger M runs the tiled kernel.  Both
 * compute the exact integer product, so the choice never changes a result. */

/* hbl_gemm_s32 — the integer product acc = q . t^T (exact), for inspection and tests.
 *  codes [M, K*abits/8], Wq [N, K/4], acc [M, N] int32 row-major.  N >= 1. */
hbl_status hbl_gemm_s32(const uint8_t* codes, const uint8_t* Wq, int64_t M, int64_t K, int64_t N,
                        int abits, int32_t* acc, void* stream);

/* hbl_gemm_dequant — integer product plus the dequantisation epilogue
 *  y[m,n] = fl32(fl32((float)acc[m,n] * deq[m]) * (*w_scale)), y [M, N] fp32 row-major. */
hbl_status hbl_gemm_dequant(const uint8_t* codes, const float* deq, const uint8_t* Wq,
                            const float* w_scale, int64_t M, int64_t K, int64_t N, int abits, float* y,
                            void* stream);

/* hbl_forward — the whole H-BitLinear (use_hadamard = 1) or BitLinear (use_hadamard = 0)
 * forward: hbl_quantize_activations into the workspace, then hbl_gemm_dequant into y.
 *  ws  at least hbl_forward_workspace_bytes(M, K, abits) bytes of device memory. */
hbl_status hbl_forward(const void* x, hbl_dtype xt, const uint8_t* Wq, const float* w_scale, int64_t M,
                       int64_t K, int64_t N, int abits, int use_hadamard, hbl_norm norm,
                       const float* gamma, float norm_eps, float* y, void* ws, size_t ws_bytes,
                       void* stream);

/* The activation statistic switch.  The write-up (section H-BitLinear模塊) says INT8 and INT4
 * activations use different strategies and drops both equations; HBL_STAT_ABSMAX (the
 * default of every other call) is the reading above, HBL_STAT_ABSMEAN the alternative for
 * INT4: the absmean function the pages give for the weights (scale by the mean absolute
 * value, round to the nearest integer, clip) on the INT4 grid:
 *     b = (float)((sum_k |z_k|, fp64) / K); if b < 2^-120: q = 0, deq = 0
 *     else: s = fl32(1 / b);  q = clamp(rint_ne(fl32(z * s)), -8, 7);  deq = fl32(fl32(b * r) * hK)
 * Codes, packing and the GEMM are unchanged.  HBL_STAT_ABSMEAN needs abits = 4
 * (HBL_ERR_UNSUPPORTED otherwise).  The sum's order on the GPU differs from ascending; b can
 * differ from the ascending-order value by one ulp in rare rows (about 1e-5 of rows), which
 * moves codes at rounding boundaries. */
hbl_status hbl_quantize_activations_stat(const void* x, hbl_dtype xt, int64_t M, int64_t K, hbl_norm norm,
                                         const float* gamma, float norm_eps, int abits, int use_hadamard, int stat,
                                         uint8_t* codes, float* deq, void* stream);
hbl_status hbl_forward_stat(const void* x, hbl_dtype xt, const uint8_t* Wq, const float* w_scale, int64_t M,
                            int64_t K, int64_t N, int abits, int use_hadamard, hbl_norm norm, const float* gamma,
                            float norm_eps, int stat, float* y, void* ws, size_t ws_bytes, void* stream);

/* hbl_forward_noalloc — hbl_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The same
 * kernels and results as hbl_forward, bit for bit, but the codes and deq of the call live in
 * a static device array of HBL_NOALLOC_SCRATCH_BYTES that the library owns: one per GPU, on
 * the device current at the call (the stream must belong to it), set up by the first call on
 * that device and kept until the process ends.  The call allocates nothing.
 *  Needs hbl_forward_workspace_bytes(M, K, abits) <= HBL_NOALLOC_SCRATCH_BYTES
 *  (HBL_ERR_UNSUPPORTED otherwise, before any HIP call): e.g. M = 8192, K = 16384 at abits 4.
 *  Calls on one GPU share its array: calls that overlap in time on that GPU (several streams,
 *  or several host threads) race on it and must be ordered by the caller.  The array keeps
 *  the last call's codes and deq; every call writes all it reads, so nothing needs clearing. */
#define HBL_NOALLOC_SCRATCH_BYTES (80u << 20)
hbl_status hbl_forward_noalloc(const void* x, hbl_dtype xt, const uint8_t* Wq, const float* w_scale, int64_t M,
                               int64_t K, int64_t N, int abits, int use_hadamard, hbl_norm norm, const float* gamma,
                               float norm_eps, float* y, void* stream);

/* 1 if hbl_forward(M, K, ..., abits, use_hadamard) runs as one fused kernel, else 0.  With a
 * few token rows (use_hadamard, K = 4096 .. 16384, M <= 256 / (K / 64)), each block of the
 * decode GEMM transforms and quantises the rows itself while its weights stream in; results
 * (y, and the codes and deq left in the workspace) are identical to the two-kernel path. */
int hbl_forward_fused(int64_t M, int64_t K, int abits, int use_hadamard);

/* hbl_swiglu — the FFN gate of the LLaMA-like block (write-up section
 * "BitNet v2：原生4位激活": RMSNorm, SwishGLU, no bias):
 *  h[i] = fl32( silu(g[i]) * u[i] ),  silu(v) = v / (1 + exp(-v)) in fp32.
 *  g, u, h: n fp32 each; h may alias neither g nor u.  n >= 0. */
hbl_status hbl_swiglu(const float* g, const float* u, int64_t n, float* h, void* stream);

/* ---- FFN block ---------------------------------------------------------------------------
 * The LLaMA-like FFN of BitNet v2 (write-up section "BitNet v2：原生4位激活": RMSNorm,
 * SwishGLU, no biases; section H-BitLinear模塊: only the down projection takes the Hadamard
 * transform, gate and up are plain BitLinear):
 *     codes, deq = quantize_activations(x, RMS with gamma_in, no transform)   (shared)
 *     g = gemm_dequant(codes, deq, Wq_gate, scale_gate)                     [M, F]
 *     u = gemm_dequant(codes, deq, Wq_up,   scale_up)                       [M, F]
 *     h = silu(g) * u                      (as hbl_swiglu; rounded to bf16 if ht = HBL_BF16)
 *     y = forward(h, Wq_down, scale_down, RMS with gamma_down, Hadamard over F)   [M, D]
 * Gate and up run as one GEMM over their interleaved weights whose epilogue writes only h;
 * g and u never reach memory.  Every value equals the unfused sequence of calls bit for bit. */

/* Wgu — the gate and up weights (each in the Wq format, F rows of K/4 bytes) interleaved in
 * blocks of 32 rows: rows 64b .. 64b+31 of Wgu are gate rows 32b .. 32b+31, rows 64b+32 ..
 * 64b+63 the up rows 32b .. 32b+31.  F % 32 == 0.  Size 2*F*K/4 bytes (0 if invalid). */
size_t hbl_packed_gate_up_bytes(int64_t F, int64_t K);
/* Builds Wgu from two packed weights (two strided device copies on the stream); no overlap. */
hbl_status hbl_interleave_gate_up(const uint8_t* Wq_gate, const uint8_t* Wq_up, int64_t F, int64_t K, uint8_t* Wgu,
                                  void* stream);
/* h [M, F] (fp32 or bf16 by ht) = silu(g) * u with g, u as hbl_gemm_dequant of the shared
 * codes [M, K*abits/8] / deq [M] with the gate (scale_gate) and up (scale_up) halves of Wgu. */
hbl_status hbl_gate_up_swiglu(const uint8_t* codes, const float* deq, const uint8_t* Wgu, const float* scale_gate,
                              const float* scale_up, int64_t M, int64_t K, int64_t F, int abits, hbl_dtype ht, void* h,
                              void* stream);
/* Workspace of hbl_ffn_forward: input codes + deq, h, and the down projection's codes + deq. */
size_t hbl_ffn_workspace_bytes(int64_t M, int64_t D, int64_t F, int abits, hbl_dtype ht);
/* The whole block: x [M, D] (xt) -> y [M, D] fp32.  D % 64 == 0; F a power of two in
 * [64, HBL_MAX_K_HADAMARD]; gamma_in [D] / gamma_down [F] or NULL for unit gamma; ht is the
 * storage type of h; the same abits for both quantisations. */
hbl_status hbl_ffn_forward(const void* x, hbl_dtype xt, const uint8_t* Wgu, const float* scale_gate,
                           const float* scale_up, const uint8_t* Wq_down, const float* scale_down, int64_t M, int64_t D,
                           int64_t F, int abits, const float* gamma_in, const float* gamma_down, float norm_eps,
                           hbl_dtype ht, float* y, void* ws, size_t ws_bytes, void* stream);

/* ---- FP6 x FP4 a4 path ----------------------------------------------------------------
 * The same layer with the a4 codes stored as FP6 and the weights as FP4 (formats above);
 * outputs are bit-identical to the INT4 / 2-bit calls.  Written for the 4-bit matrix
 * hardware the BitNet v2 write-up motivates a4 with (section "原生4比特計算"). */
size_t hbl_packed_weight_fp4_bytes(int64_t N, int64_t K);         /* N*K/2          */
size_t hbl_packed_act_fp6_bytes(int64_t M, int64_t K);            /* M*K*3/4        */
size_t hbl_forward_fp6fp4_workspace_bytes(int64_t M, int64_t K);

/* Wq (2-bit, from hbl_quantize_weights) -> Wq4 [N, K/2] FP4.  w_scale is unchanged. */
hbl_status hbl_weights_to_fp4(const uint8_t* Wq, int64_t N, int64_t K, uint8_t* Wq4, void* stream);

/* As hbl_quantize_activations with abits = 4, writing codes6 [M, 3K/4] instead of nibbles. */
hbl_status hbl_quantize_activations_fp6(const void* x, hbl_dtype xt, int64_t M, int64_t K, hbl_norm norm,
                                        const float* gamma, float norm_eps, int use_hadamard, uint8_t* codes6,
                                        float* deq, void* stream);

/* Integer product of codes6 and Wq4 (exact; acc [M, N] int32), and with the dequant epilogue
 * (y [M, N] fp32, same association as hbl_gemm_dequant). */
hbl_status hbl_gemm_fp6fp4_s32(const uint8_t* codes6, const uint8_t* Wq4, int64_t M, int64_t K, int64_t N,
                               int32_t* acc, void* stream);
hbl_status hbl_gemm_fp6fp4_dequant(const uint8_t* codes6, const float* deq, const uint8_t* Wq4,
                                   const float* w_scale, int64_t M, int64_t K, int64_t N, float* y,
                                   void* stream);

/* The whole a4 forward on the FP6 x FP4 path; ws >= hbl_forward_fp6fp4_workspace_bytes(M, K). */
hbl_status hbl_forward_fp6fp4(const void* x, hbl_dtype xt, const uint8_t* Wq4, const float* w_scale, int64_t M,
                              int64_t K, int64_t N, int use_hadamard, hbl_norm norm, const float* gamma,
                              float norm_eps, float* y, void* ws, size_t ws_bytes, void* stream);

/* ---- QKV states (low-bit attention) -----------------------------------------------------
 * The BitNet v2 write-up (text of Tables 2 and 3) quantises the Q, K and V states after RoPE,
 * each head directly to unsigned integers with the absmax function and no calibration data,
 * and keeps the KV cache at 3 bits.  Reading implemented here, per head vector x of length d
 * (one row per token and head, post-RoPE, supplied by the caller), L = 2^bits - 1:
 *     g = max|x|,  s = fl32(L / fl32(2g)) (s = 0 if g < 2^-120),  c = L/2,
 *     u = clamp(rint_ne(fl32(fl32(x*s) + c)), 0, L)
 * so [-g, g] maps onto 0 .. L with both ends reachable.  Inverse:
 *     xhat = fl32(fl32(u - c) * fl32(fl32(2g) / L)).
 * codes — rows of d*bits/8 bytes; code i of a row at bits [bits*i, bits*i + bits) of the row
 *     read as a little-endian bit string.  gamma — one fp32 g per row.
 * Limits: d in {32, 64, 128, 256, 512}; 2 <= bits <= 8. */
size_t hbl_packed_qkv_bytes(int64_t rows, int64_t d, int bits);   /* rows*d*bits/8 */
hbl_status hbl_quantize_qkv(const void* x, hbl_dtype xt, int64_t rows, int64_t d, int bits, uint8_t* codes,
                            float* gamma, void* stream);
hbl_status hbl_dequantize_qkv(const uint8_t* codes, const float* gamma, int64_t rows, int64_t d, int bits, float* out,
                              void* stream);

/* Static text for a status code, and the detail of the last failure on this thread. */
const char* hbl_status_string(hbl_status s);
const char* hbl_last_error(void);
/* Library version: major*10000 + minor*100 + patch. */
int hbl_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HBL_H_ */
