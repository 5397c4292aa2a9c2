// Per-token int8 activation quantisation for the W4A8 path.
//
// "What this repo does that stock vLLM doesn't", "In full" item 4: the W4A8
// path keeps the int4 weights and quantises activations to int8 per token.
// Per row m:  scale = fp32(max|x|) / 127 (IEEE division),
//             q = clamp(rne(fp32(x) / scale), -127, 127);  a zero row -> 0, 0.
//
// HBM-bound (2 bytes in, 1 byte out per element).  A row is held in registers
// between the absmax pass and the quantise pass, so x is read from HBM once.
// One workgroup per row, with as many threads (up to 1024) as it takes to
// give each a few 16-byte chunks; rows longer than the register budget are
// re-read (from cache) in the quantise pass.
//
// Division.  The quotient x / scale is formed without a divide per element:
// with r = 1 / scale (one IEEE division per thread), y0 = x * r,
// e = fma(-y0, scale, x) (exact residual) and y1 = fma(e, r, y0).  Markstein's
// correction step makes y1 the correctly rounded quotient here; an exhaustive
// run over every finite fp16 absmax and every fp16 x with |x| <= absmax
// (1,007,713,278 pairs) gave rint(y1) == rint(x / scale) in all of them.
//
// Output orders.  Row-major q[m][k], and/or the "fragment" order the
// weight-streaming W4A8 GEMM loads: rows in tiles of 16, and for tile mt,
// group g, half h (64 k) a 1 KiB block at byte ((mt*G + g)*2 + h) * 1024 in
// which lane l = col + 16*quad owns the 16 codes of row 16*mt + col at
// k = 128 g + 64 h + 16 quad + [0, 16).  That is exactly one 16-byte operand
// of v_mfma_i32_16x16x64_i8 per lane, so the GEMM moves it with one
// contiguous 1 KiB load.  Rows of the last tile past M are left unwritten
// (the GEMM never stores their results).
#include <algorithm>

#include "common.h"

namespace qg {
namespace {

// |x| maximum of 8 fp16 values, as float.  The sign bit is cleared and the
// remaining 15-bit patterns compared as unsigned integers: for finite fp16,
// magnitude order equals bit-pattern order.
__device__ __forceinline__ uint32_t absmax_bits8(uint4 v) {
  uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu, c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
  uint32_t m0 = max(a & 0xFFFFu, a >> 16), m1 = max(b & 0xFFFFu, b >> 16);
  uint32_t m2 = max(c & 0xFFFFu, c >> 16), m3 = max(d & 0xFFFFu, d >> 16);
  return max(max(m0, m1), max(m2, m3));
}

// rint(x / s) clamped to [-127, 127], with rs = 1 / s (see "Division").
__device__ __forceinline__ int quant1(uint32_t hbits, float s, float rs) {
  const float x = half_bits_to_float(hbits);
  const float y0 = x * rs;
  const float e = __builtin_fmaf(-y0, s, x);
  const float y1 = __builtin_fmaf(e, rs, y0);
  return (int)fminf(fmaxf(rintf(y1), -127.0f), 127.0f);
}

__device__ __forceinline__ uint2 quant8(uint4 v, float s, float rs) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = (uint32_t)(quant1(w[i] & 0xFFFFu, s, rs) & 0xFF);
    uint32_t hi = (uint32_t)(quant1(w[i] >> 16, s, rs) & 0xFF);
    out[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
  }
  return make_uint2(out[0], out[1]);
}

// The workgroup's blockDim.x threads cooperate on one row; each holds up to
// MAXC 16-byte chunks (8 fp16 values) in registers.  Chunks past
// blockDim.x * MAXC are re-read from memory in the quantise pass (only for
// very long rows).
template <int MAXC>
__global__ __launch_bounds__(1024) void act_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx, int K,
                                                         int8_t* __restrict__ q, int64_t ldq,
                                                         int8_t* __restrict__ qfrag, float* __restrict__ scale) {
  const int T = (int)blockDim.x;
  const int t = (int)threadIdx.x;
  const int64_t m = blockIdx.x;
  const uint16_t* row = x + m * ldx;
  const int nch = K >> 3;

  uint4 v[MAXC];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + T * i;
    if (c < nch) {
      v[i] = *reinterpret_cast<const uint4*>(row + 8 * c);
      amax = max(amax, absmax_bits8(v[i]));
    } else {
      v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  for (int c = t + T * MAXC; c < nch; c += T)
    amax = max(amax, absmax_bits8(*reinterpret_cast<const uint4*>(row + 8 * c)));

  float a = wave_max(half_bits_to_float(amax));
  if (T > kWave) {
    __shared__ float red[1024 / kWave];
    if ((t & 63) == 0) red[t >> 6] = a;
    __syncthreads();
    for (int i = 0; i < T / kWave; ++i) a = fmaxf(a, red[i]);
  }

  const float s = a / 127.0f;   // IEEE fp32 division
  const float rs = 1.0f / s;    // IEEE fp32 division, once per thread
  if (t == 0) scale[m] = a > 0.0f ? s : 0.0f;
  const int G = K / kGroup;
  const int mt = (int)(m >> 4), col = (int)(m & 15);
  // stores the 8 codes of chunk c (k = 8c .. 8c+7) in the requested orders
  auto put = [&](int c, uint2 codes) {
    if (q) *reinterpret_cast<uint2*>(q + m * ldq + 8 * c) = codes;
    if (qfrag) {
      const int k = 8 * c, g = k >> 7, kk = k & 127, h = kk >> 6, quad = (kk & 63) >> 4;
      const int64_t off = ((((int64_t)mt * G + g) * 2 + h) * 64 + col + 16 * quad) * 16 + (kk & 15);
      *reinterpret_cast<uint2*>(qfrag + off) = codes;
    }
  };
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + T * i;
    if (c < nch) put(c, a > 0.0f ? quant8(v[i], s, rs) : make_uint2(0, 0));
  }
  for (int c = t + T * MAXC; c < nch; c += T)
    put(c, a > 0.0f ? quant8(*reinterpret_cast<const uint4*>(row + 8 * c), s, rs) : make_uint2(0, 0));
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                            int64_t ldq, int8_t* qfrag, float* scale, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  // One workgroup per row: the fewest chunks per thread (1, 2, 3, 4 or 8;
  // longer rows re-read) that fit 1024 threads, then just enough waves.
  const int64_t nch = K / 8;
  int maxc = (int)((nch + 1023) / 1024);
  maxc = maxc <= 4 ? maxc : 8;
  const int64_t per = (nch + maxc - 1) / maxc;
  const unsigned threads = (unsigned)std::min<int64_t>(1024, (per + 63) / 64 * 64);
  const dim3 grid((unsigned)M);
  switch (maxc) {
    case 1: act_quant_kernel<1><<<grid, threads, 0, st>>>(x, ldx, (int)K, q, ldq, qfrag, scale); break;
    case 2: act_quant_kernel<2><<<grid, threads, 0, st>>>(x, ldx, (int)K, q, ldq, qfrag, scale); break;
    case 3: act_quant_kernel<3><<<grid, threads, 0, st>>>(x, ldx, (int)K, q, ldq, qfrag, scale); break;
    case 4: act_quant_kernel<4><<<grid, threads, 0, st>>>(x, ldx, (int)K, q, ldq, qfrag, scale); break;
    default: act_quant_kernel<8><<<grid, threads, 0, st>>>(x, ldx, (int)K, q, ldq, qfrag, scale); break;
  }
  return hipGetLastError();
}

}  // namespace qg
