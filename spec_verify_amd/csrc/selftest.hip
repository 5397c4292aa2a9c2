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
#include <type_traits>

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


// Load floors.  A diagnostic read with the access pattern of a weight-
// streaming kernel and none of its arithmetic: workgroup b reads slice
// lin / share of a (a's bytes dealt into wgs / share slices) and slice
// lin % share of c (c's bytes dealt into share slices), where lin is b
// walked as in the row-split decode GEMM (the `share` workgroups that read
// one slice of a are consecutive on one XCD).  Each thread reads its 16-byte
// chunks 16 at a time (its slice of a, then its slice of c) with range-
// checked buffer loads and folds them into a checksum, one word per wave,
// so that no load is dead.
template <bool NT>
__global__ __launch_bounds__(1024) void probe_read_kernel(const uint8_t* a, int64_t a_bytes, const uint8_t* c,
                                                          int64_t c_bytes, int share, uint32_t* sink) {
  const unsigned total = gridDim.x, per = total >> 3;
  unsigned lin = blockIdx.x;
  if ((total & 7u) == 0 && per % (unsigned)share == 0) lin = (blockIdx.x & 7u) * per + (blockIdx.x >> 3);
  const int64_t na = (int64_t)total / share, sa = (int64_t)(lin / (unsigned)share), sc = (int64_t)(lin % (unsigned)share);
  const int64_t a0 = a_bytes * sa / na, a1 = a_bytes * (sa + 1) / na;
  const int64_t c0 = c_bytes * sc / share, c1 = c_bytes * (sc + 1) / share;
  uint32_t acc = 0;
  auto walk = [&](const uint8_t* base, int64_t lo, int64_t hi, auto nt) {
    if (hi <= lo) return;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + lo), (short)0, (int)(hi - lo), 0x00020000);
    const int64_t n16 = (hi - lo + 15) / 16;
    for (int64_t i = threadIdx.x; i < n16; i += (int64_t)blockDim.x * 16) {
      uint4 v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t k = i + (int64_t)blockDim.x * j;
        const uint32_t off = k < n16 ? (uint32_t)(k * 16) : 0x80000000u;   // past the slice: reads zeros
        v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, decltype(nt)::value ? 2 : 0));
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
  };
  walk(a, a0, a1, std::integral_constant<bool, NT>{});
  walk(c, c0, c1, std::false_type{});
  // one word per wave: its lanes' checksums folded together
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_quant_division_check(unsigned long long* counts, hipStream_t st) {
  quant_division_check_kernel<<<dim3(kMaxFiniteHalf), dim3(256), 0, st>>>(counts);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* a, int64_t a_bytes, const void* c, int64_t c_bytes, int share, int wgs,
                             int threads, bool nt, uint32_t* sink, hipStream_t st) {
  const uint8_t* pa = reinterpret_cast<const uint8_t*>(a);
  const uint8_t* pc = reinterpret_cast<const uint8_t*>(c);
  if (nt)
    probe_read_kernel<true><<<dim3((unsigned)wgs), dim3((unsigned)threads), 0, st>>>(pa, a_bytes, pc, c_bytes, share, sink);
  else
    probe_read_kernel<false><<<dim3((unsigned)wgs), dim3((unsigned)threads), 0, st>>>(pa, a_bytes, pc, c_bytes, share, sink);
  return hipGetLastError();
}

}  // namespace qg
