// plan.cpp — host-only dispatch decisions of the C ABI layer (no kernels, no HIP calls), kept
// apart from the kernel sources so that the argument-validation layer can also be built and
// tested on its own on a host without a GPU.
#include "hbl_internal.h"

namespace hbl {

// The fused decode kernel covers the transform over K = 2^12 .. 2^14 with at most
// DEC_MAX_GROUPS groups of R = 256 / (K / 64) rows (one 256-thread block transforms R rows).
bool decode_fused_ok(int64_t M, int64_t K, int abits, int use_h) {
  if (!use_h || (abits != 4 && abits != 8) || M < 1) return false;
  int L = 0;
  while ((int64_t(1) << L) < K) ++L;
  if (L < 12 || L > 14) return false;
  const int64_t R = (int64_t)256 / ((int64_t(1) << L) / 64);
  return M <= DEC_MAX_GROUPS * R;
}

}  // namespace hbl
