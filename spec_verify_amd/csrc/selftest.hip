// Exhaustive device self-test of the quantiser's division.
//
// The per-token quantiser ("What this repo does that stock vLLM doesn't",
// "In full" item 4: activations quantised to int8 per token, here with
// scale = absmax / 127 and codes rint(x / scale)) replaces the per-element
// IEEE division by a reciprocal product with one correction step
// (corrected_quotient).  This kernel runs that step and the IEEE division
// side by side over every finite positive fp16 absmax a (bit patterns
// 0x0001 .. 0x7BFF) and every fp16 x with |x| <= a, zeros of both signs
// included, and counts the pairs whose rounded quotients differ.
#include "common.h"
#include "quant_math.h"

namespace qg {
namespace {

constexpr uint32_t kMaxFiniteHalf = 0x7BFFu;

__global__ __launch_bounds__(256) void quant_division_check_kernel(unsigned long long* counts) {
  const uint32_t abits = blockIdx.x + 1u;            // 0x0001 .. 0x7BFF
  const float a = half_bits_to_float(abits);
  const float s = a / 127.0f;                        // IEEE, as in the quantiser
  const float rs = 1.0f / s;
  unsigned long long pairs = 0, bad = 0;
  // x = +0 .. +a (bits 0 .. abits) and -0 .. -a (bits 0x8000 .. 0x8000 | abits)
  for (uint32_t i = threadIdx.x; i <= 2u * abits + 1u; i += blockDim.x) {
    const uint32_t xb = i <= abits ? i : 0x8000u | (i - abits - 1u);
    const float x = half_bits_to_float(xb);
    const float want = rintf(x / s);                 // IEEE division
    const float got = rintf(corrected_quotient(x, s, rs));
    ++pairs;
    bad += (want != got) ? 1u : 0u;
  }
  atomicAdd(&counts[0], pairs);
  if (bad) atomicAdd(&counts[1], bad);
}

}  // namespace

hipError_t launch_quant_division_check(unsigned long long* counts, hipStream_t st) {
  quant_division_check_kernel<<<dim3(kMaxFiniteHalf), dim3(256), 0, st>>>(counts);
  return hipGetLastError();
}

}  // namespace qg
