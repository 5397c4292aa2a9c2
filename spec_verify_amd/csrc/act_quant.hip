// Per-token int8 activation quantisation for the W4A8 path.
//
// "What this repo does that stock vLLM doesn't", "In full" item 4: the W4A8
// path keeps the int4 weights and quantises activations to int8 per token.
// Per row m:  scale = fp32(max|x|) / 127 (IEEE division),
//             q = clamp(rne(fp32(x) / scale), -127, 127);  a zero row -> 0, 0.
//
// HBM-bound (2 bytes in, 1 byte out per element).  A row is held in registers
// between the absmax pass and the quantise pass, so x is read from HBM once.
// One 256-thread workgroup per row; rows longer than the register budget are
// re-read (from cache) in the quantise pass.
//
// Output orders.  Row-major q[m][k], and/or the "fragment" order the
// weight-streaming W4A8 GEMM loads: rows in tiles of 16, and for tile mt,
// group g, half h (64 k) a 1 KiB block at byte ((mt*G + g)*2 + h) * 1024 in
// which lane l = col + 16*quad owns the 16 codes of row 16*mt + col at
// k = 128 g + 64 h + 16 quad + [0, 16).  That is exactly one 16-byte operand
// of v_mfma_i32_16x16x64_i8 per lane, so the GEMM moves it with one
// contiguous 1 KiB load.  Rows of the last tile past M are left unwritten
// (the GEMM never stores their results).
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

__device__ __forceinline__ int quant1(uint32_t hbits, float s) {
  float xf = half_bits_to_float(hbits);
  float r = rintf(xf / s);                 // correctly rounded fp32 divide, then ties-to-even
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ uint2 quant8(uint4 v, float s) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = (uint32_t)(quant1(w[i] & 0xFFFFu, s) & 0xFF);
    uint32_t hi = (uint32_t)(quant1(w[i] >> 16, s) & 0xFF);
    out[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
  }
  return make_uint2(out[0], out[1]);
}

// THREADS threads cooperate on one row; each holds up to MAXC 16-byte chunks
// (8 fp16 values) in registers.  Chunks past THREADS*MAXC are re-read from
// memory in the quantise pass (only for very long rows).
template <int THREADS, int MAXC>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                        int K, int64_t M, int8_t* __restrict__ q,
                                                        int64_t ldq, int8_t* __restrict__ qfrag,
                                                        float* __restrict__ scale) {
  constexpr int ROWS = 256 / THREADS;
  const int t = threadIdx.x % THREADS;
  const int64_t m = (int64_t)blockIdx.x * ROWS + threadIdx.x / THREADS;
  const bool live = m < M;
  const uint16_t* row = x + (live ? m : 0) * ldx;
  const int nch = K >> 3;

  uint4 v[MAXC];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + THREADS * i;
    if (live && c < nch) {
      v[i] = *reinterpret_cast<const uint4*>(row + 8 * c);
      amax = max(amax, absmax_bits8(v[i]));
    } else {
      v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  for (int c = t + THREADS * MAXC; live && c < nch; c += THREADS)
    amax = max(amax, absmax_bits8(*reinterpret_cast<const uint4*>(row + 8 * c)));

  float a = wave_max(half_bits_to_float(amax));
  if constexpr (THREADS > kWave) {
    __shared__ float red[256 / kWave];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < THREADS / kWave; ++i) a = fmaxf(a, red[i]);
  }
  if (!live) return;

  const float s = a / 127.0f;   // IEEE fp32 division
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
    const int c = t + THREADS * i;
    if (c < nch) put(c, a > 0.0f ? quant8(v[i], s) : make_uint2(0, 0));
  }
  for (int c = t + THREADS * MAXC; c < nch; c += THREADS)
    put(c, a > 0.0f ? quant8(*reinterpret_cast<const uint4*>(row + 8 * c), s) : make_uint2(0, 0));
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                            int64_t ldq, int8_t* qfrag, float* scale, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int nch = (int)(K / 8);
  // One 256-thread workgroup per row: a few 16-byte chunks per thread keep
  // many rows' loads in flight and the divides spread over more waves.
  const dim3 grid((unsigned)M);
  if (nch <= 256 * 4)
    act_quant_kernel<256, 4><<<grid, 256, 0, st>>>(x, ldx, (int)K, M, q, ldq, qfrag, scale);
  else if (nch <= 256 * 12)
    act_quant_kernel<256, 12><<<grid, 256, 0, st>>>(x, ldx, (int)K, M, q, ldq, qfrag, scale);
  else
    act_quant_kernel<256, 24><<<grid, 256, 0, st>>>(x, ldx, (int)K, M, q, ldq, qfrag, scale);
  return hipGetLastError();
}

}  // namespace qg
