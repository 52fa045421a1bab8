// hbl_internal.h — launchers implemented by the kernel translation units and called by
// the C ABI layer (api.cpp) after argument validation.  Each returns hipSuccess or the
// launch error.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hbl {

// Weight ternarisation (k_wquant.hip).  ws: N doubles.
hipError_t launch_wquant(const float* W, int64_t N, int64_t K, uint8_t* Wq, float* w_scale, double* ws,
                         hipStream_t s);

// Activation quantisation (k_actquant.hip).  xt: 0 fp32, 1 bf16.  abits: 4 (INT4 nibbles),
// 8 (INT8), 6 (INT4 values stored as FP6 E2M3 codes) or 5 (INT4 nibbles with the absmean
// statistic).
hipError_t launch_actquant(const void* x, int xt, int64_t M, int64_t K, int norm, const float* gamma,
                           float eps, int abits, int use_h, uint8_t* codes, float* deq, hipStream_t s);

// bf16 rows with unit gamma and K = 2^10 .. 2^14 under the transform take the activation
// kernel that runs five or six transform stages on the matrix cores (k_actquant_mfma.hip);
// launch_actquant dispatches to it.  abits as launch_actquant.
bool actquant_mfma_ok(int xt, int64_t K, const float* gamma, int norm, int use_h);
hipError_t launch_actquant_mfma(const void* x, int64_t M, int64_t K, int norm, float eps, int abits, uint8_t* codes,
                                float* deq, hipStream_t s);

// The whole H-BitLinear forward for a few token rows in one kernel (k_actquant.hip): applies
// when decode_fused_ok(M, K, abits, use_h) (plan.cpp); writes codes/deq (workspace) and y like
// the two-kernel path, bit for bit.  One group of R = 256 / (K / 64) rows (the rows one block
// transforms at once): with more rows the two-kernel path is faster.
constexpr int DEC_MAX_GROUPS = 1;
bool decode_fused_ok(int64_t M, int64_t K, int abits, int use_h);
hipError_t launch_decode_fused(const void* x, int xt, int64_t M, int64_t K, int norm, const float* gamma, float eps,
                               int abits, const uint8_t* Wq, const float* w_scale, int64_t N, uint8_t* codes,
                               float* deq, float* y, hipStream_t s);

// Integer GEMM with either an int32 output (acc != nullptr) or the dequantising epilogue
// (y != nullptr) (k_gemm.hip).
hipError_t launch_gemm(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale,
                       int64_t M, int64_t K, int64_t N, int abits, int32_t* acc, float* y, hipStream_t s);

// Tile size and K splits of the tiled GEMMs (k_gemm.hip): 256 x 256 tiles (big) or 128 x 128,
// and the number of blocks that share each tile's K (their int32 results added atomically);
// below the big tiles, 64 x 128 tiles run unsplit instead where small_tiles_unsplit holds.
constexpr int64_t CUS = 256;
struct GemmPlan {
  bool big;
  int splits;
};
bool use_big_tiles(int64_t M, int64_t N);
bool small_tiles_unsplit(int64_t M, int64_t N, int64_t K);
GemmPlan plan_tiles(int64_t M, int64_t N, int64_t K);
// Split-K helpers (k_gemm.hip): zero n int32, and dequantise an int32 product in place
// (y[m, n] = fl(fl((float)acc[m, n] * deq[m]) * w_scale[0]), same bits as the epilogue).
hipError_t launch_zero32(int32_t* p, int64_t n, hipStream_t s);
hipError_t launch_dequant32(void* buf, const float* deq, const float* w_scale, int64_t M, int64_t N, hipStream_t s);

// The same GEMM with its tiles loaded straight into LDS (k_gemm_dma.hip), for K a multiple of
// the stage depth (gemm_dma_ok): tile 256 runs 256 x 256 tiles (mode 0: int32 acc, 1: dequant),
// tile 64 runs 64 x 128 tiles, any other value 128 x 256 tiles; modes 2 and 3 are the fused
// gate/up epilogue (out: h as fp32 / bf16, N = 2F interleaved rows).  Same int32 sums and
// output bits as launch_gemm.
bool gemm_dma_ok(int64_t K, int abits);
hipError_t launch_gemm_dma(int tile, int mode, const uint8_t* codes, const float* deq, const uint8_t* Wq,
                           const float* w_scale, const float* w_scale_up, int64_t M, int64_t K, int64_t N, int abits,
                           int32_t* acc, void* out, hipStream_t s);

// Decode-regime GEMM for M <= GEMV_MAX_M token rows (k_gemv.hip); launch_gemm dispatches to it.
constexpr int64_t GEMV_MAX_M = 64;
hipError_t launch_gemv(const uint8_t* codes, const float* deq, const uint8_t* Wq, const float* w_scale,
                       int64_t M, int64_t K, int64_t N, int abits, int32_t* acc, float* y, hipStream_t s);

// Fused FFN gate/up projection (k_gemm.hip): Wgu holds 2F rows, gate and up interleaved in
// blocks of 32; h [M, F] = silu(g) * u stored as fp32 (h_bf16 = 0) or bf16 (h_bf16 = 1).
hipError_t launch_gemm_swiglu(const uint8_t* codes, const float* deq, const uint8_t* Wgu, const float* scale_gate,
                              const float* scale_up, int64_t M, int64_t K, int64_t F, int abits, int h_bf16, void* h,
                              hipStream_t s);

// GEMM of FP6-coded INT4 activations with FP4-coded ternary weights (k_gemm_f6f4.hip).
hipError_t launch_gemm_f6f4(const uint8_t* codes6, const float* deq, const uint8_t* Wq4, const float* w_scale,
                            int64_t M, int64_t K, int64_t N, int32_t* acc, float* y, hipStream_t s);
// 2-bit ternary words -> FP4 E2M1 nibbles (k_gemm_f6f4.hip).
hipError_t launch_weights_fp4(const uint8_t* Wq, int64_t N, int64_t K, uint8_t* Wq4, hipStream_t s);

// Unsigned absmax quantisation of head vectors and its inverse (k_qkv.hip); d in
// {32, 64, 128, 256, 512}, bits in 2..8, xt 0 fp32 / 1 bf16.
hipError_t launch_qkv_quant(const void* x, int xt, int64_t rows, int64_t d, int bits, uint8_t* codes, float* gamma,
                            hipStream_t s);
hipError_t launch_qkv_dequant(const uint8_t* codes, const float* gamma, int64_t rows, int64_t d, int bits, float* out,
                              hipStream_t s);

// h = silu(g) * u (k_swiglu.hip).
hipError_t launch_swiglu(const float* g, const float* u, int64_t n, float* h, hipStream_t s);

}  // namespace hbl
