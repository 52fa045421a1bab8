// k_actquant_mfma.hip — the H-BitLinear activation kernel for bf16 rows (K = 2^10 .. 2^14, unit
// gamma): load -> RMSNorm statistics -> online fast Walsh-Hadamard transform with five or six
// of its stages on the matrix cores (actquant_mfma.h) -> per-token absmax (or absmean) ->
// INT4/INT8 codes (or INT4 codes stored as FP6) + one dequant factor per row.
//
// BitNet v2 write-up, section H-BitLinear模塊: LN, then the online Hadamard transform by the
// fast Hadamard transform, then per-token INT8/INT4 quantisation.  bitnet.cpp article, section
// "6 页论文，引入 1 bit LLM": activations are scaled into [-Qb, Qb] without a zero point.
//
// Blocks are persistent (two resident per CU); each walks slabs of 16384 elements and loads the
// next slab into the raw registers as soon as the matrix cores have read the current one.  The
// RMSNorm factor r and 1/sqrt(K) are folded into deq: absmax codes do not change under a
// positive per-row scale.
#include <cmath>

#include "actquant_mfma.h"
#include "actquant_store.h"
#include "hbl_device.h"
#include "hbl_internal.h"

namespace hbl {
namespace {

template <int L, int ABITS, int NM>
__global__ __launch_bounds__(HM_WG) void k_actquant_hm(const uint16_t* __restrict__ x, int64_t M, float eps,
                                                      float hK, uint8_t* __restrict__ codes, float* __restrict__ deq) {
  constexpr int K = 1 << L;
  constexpr int R = HM_SLAB / K;   // rows per slab
  constexpr float Qb = QB<ABITS>::value;
  using P = HmPost<L>;
  __shared__ __attribute__((aligned(16))) float lds[HM_LDS_FLOATS];
  __shared__ float redf[4];
  __shared__ double redd[4];
  __shared__ double redd2[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t nslabs = (M + R - 1) / R;
  const bf16x8_t hb0 = hm_hadamard_b(lane, 0), hb1 = hm_hadamard_b(lane, 1);
  const int E0 = P::thread_E(w, lane);   // this thread's element bits outside its registers

  // One slab: transform the rows held in `cur` (reloading the next slab into `nxt` once the
  // matrix cores have read `cur`), quantise and store.  The loop below alternates two register
  // sets, so no copy is needed between slabs.
  auto slab_step = [&](uint4 (&cur)[8], uint4 (&nxt)[8], int64_t slab) __attribute__((always_inline)) {
    float v[64];
    HmStats st;
    const int64_t nslab = slab + gridDim.x;
    hm_transform<L, ABITS, NM>(cur, hb0, hb1, lds, redf, redd, redd2, w, lane, v, st, [&]() {
      if (nslab < nslabs) hm_load<L>(nxt, x, M, nslab, w, lane);
    });
    const int64_t row = slab * R + (E0 >> L);   // registers never carry row bits
    const float amax = ABITS == 5 ? (float)(st.sabs / (double)K) : st.amax;   // absmean: b = mean|z|
    // RMS factor 1/sqrt(mean(x^2) + eps): the mean in fp64, the reciprocal square root by
    // v_rsq_f32 (about one ulp; the sum of squares is already an fp32 sum per lane)
    const float r = NM != 0 ? __builtin_amdgcn_rsqf((float)(st.ss / (double)K + (double)eps)) : 1.0f;
    const bool zero = amax < 0x1p-120f;   // also keeps Qb / amax finite
    const float s = zero ? 0.0f : (ABITS == 5 ? 1.0f / amax : Qb / amax);
    if (row < M) {
      uint8_t* crow = codes + row * (int64_t)row_bytes<ABITS>(K);
#pragma unroll
      for (int g = 0; g < 64 / P::RL; ++g)
        store_run<ABITS, P::RL>(v + g * P::RL, s, crow, (E0 + P::reg_E(g * P::RL)) & (K - 1));
      if ((E0 & (K - 1)) == 0)
        deq[row] = zero ? 0.0f : __fmul_rn(__fmul_rn(ABITS == 5 ? amax : amax / Qb, r), hK);
    }
  };

  uint4 ra[8], rb[8];
  int64_t slab = blockIdx.x;
  if (slab < nslabs) hm_load<L>(ra, x, M, slab, w, lane);
  while (slab < nslabs) {
    slab_step(ra, rb, slab);
    slab += gridDim.x;
    if (slab >= nslabs) break;
    slab_step(rb, ra, slab);
    slab += gridDim.x;
  }
}

template <int L, int ABITS>
hipError_t launch_l(const void* x, int64_t M, float eps, int norm, uint8_t* codes, float* deq, hipStream_t s) {
  constexpr int K = 1 << L;
  const float hK = (float)(1.0 / std::sqrt((double)K));
  const int64_t slabs = (M + (HM_SLAB / K) - 1) / (HM_SLAB / K);
  // persistent blocks: about 71 KB of LDS each, so two are resident per CU
  const int64_t cap = 2 * CUS;
  const dim3 grid((unsigned)(slabs < cap ? slabs : cap)), block(HM_WG);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (norm)
    hipLaunchKernelGGL((k_actquant_hm<L, ABITS, 1>), grid, block, 0, s, xb, M, eps, hK, codes, deq);
  else
    hipLaunchKernelGGL((k_actquant_hm<L, ABITS, 0>), grid, block, 0, s, xb, M, eps, hK, codes, deq);
  return hipGetLastError();
}

template <int ABITS>
hipError_t dispatch(int L, const void* x, int64_t M, float eps, int norm, uint8_t* codes, float* deq, hipStream_t s) {
  switch (L) {
    case 10: return launch_l<10, ABITS>(x, M, eps, norm, codes, deq, s);
    case 11: return launch_l<11, ABITS>(x, M, eps, norm, codes, deq, s);
    case 12: return launch_l<12, ABITS>(x, M, eps, norm, codes, deq, s);
    case 13: return launch_l<13, ABITS>(x, M, eps, norm, codes, deq, s);
    case 14: return launch_l<14, ABITS>(x, M, eps, norm, codes, deq, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool actquant_mfma_ok(int xt, int64_t K, const float* gamma, int norm, int use_h) {
  return xt == 1 && use_h && (norm == 0 || gamma == nullptr) && K >= 1024 && K <= 16384 && (K & (K - 1)) == 0;
}

hipError_t launch_actquant_mfma(const void* x, int64_t M, int64_t K, int norm, float eps, int abits, uint8_t* codes,
                                float* deq, hipStream_t s) {
  if (M == 0) return hipSuccess;
  int L = 0;
  while ((int64_t(1) << L) < K) ++L;
  switch (abits) {
    case 4: return dispatch<4>(L, x, M, eps, norm, codes, deq, s);
    case 5: return dispatch<5>(L, x, M, eps, norm, codes, deq, s);
    case 6: return dispatch<6>(L, x, M, eps, norm, codes, deq, s);
    default: return dispatch<8>(L, x, M, eps, norm, codes, deq, s);
  }
}

}  // namespace hbl
