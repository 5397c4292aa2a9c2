// The quotient of the per-token int8 quantiser, shared by its kernels and
// by the library's exhaustive self-test of it.
#pragma once

#include <hip/hip_runtime.h>

namespace qg {

// x / s without a divide per element, given rs = 1 / s from one IEEE
// division: y0 = x * rs, the exact residual e = fma(-y0, s, x), and
// Markstein's correction y1 = fma(e, rs, y0).  The quantiser only needs
// rint(y1) to equal rint(x / s); that is checked exhaustively for every
// scale a / 127 of a finite fp16 absmax a and every fp16 x with |x| <= a
// (qg_selftest_quant_division).
__device__ __forceinline__ float corrected_quotient(float x, float s, float rs) {
  const float y0 = x * rs;
  const float e = __builtin_fmaf(-y0, s, x);
  return __builtin_fmaf(e, rs, y0);
}

}  // namespace qg
