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
// Division.  The quotient x / scale is formed without a divide per element
// (corrected_quotient in quant_math.h): one IEEE division per thread for
// r = 1 / scale, then a product and Markstein's correction step.  The
// library's self-test qg_selftest_quant_division runs every finite fp16
// absmax against every fp16 x with |x| <= absmax (1,007,713,278 pairs) and
// counts the pairs where rint of that quotient differs from rint of the
// IEEE quotient x / scale; a GPU test requires the count to be zero.
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
#include "quant_math.h"

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
  return (int)fminf(fmaxf(rintf(corrected_quotient(half_bits_to_float(hbits), s, rs)), -127.0f), 127.0f);
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

// Stores the 8 codes of chunk c (k = 8c .. 8c+7) of row m in the requested
// orders: row-major q (if q) and/or the fragment order (if qfrag).
__device__ __forceinline__ void put_codes(int8_t* q, int64_t ldq, int8_t* qfrag, int64_t m, int G, int c,
                                          uint2 codes) {
  if (q) *reinterpret_cast<uint2*>(q + m * ldq + 8 * c) = codes;
  if (qfrag) {
    const int mt = (int)(m >> 4), col = (int)(m & 15);
    const int k = 8 * c, g = k >> 7, kk = k & 127, h = kk >> 6, quad = (kk & 63) >> 4;
    const int64_t off = ((((int64_t)mt * G + g) * 2 + h) * 64 + col + 16 * quad) * 16 + (kk & 15);
    *reinterpret_cast<uint2*>(qfrag + off) = codes;
  }
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
  auto put = [&](int c, uint2 codes) { put_codes(q, ldq, qfrag, m, G, c, codes); };
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + T * i;
    if (c < nch) put(c, a > 0.0f ? quant8(v[i], s, rs) : make_uint2(0, 0));
  }
  for (int c = t + T * MAXC; c < nch; c += T)
    put(c, a > 0.0f ? quant8(*reinterpret_cast<const uint4*>(row + 8 * c), s, rs) : make_uint2(0, 0));
}

// ---------------------------------------------------------------------------
// RMSNorm fused with the quantiser: the norm's fp16 output y is quantised per
// row exactly as above (its codes and scale are those of act_quant on y).
//
// The norm is y = x * w / sqrt(mean(x^2) + eps), rounded to fp16.  Here it
// is evaluated in fp32, per row of length H:
//   ss = sum of x[h]^2 (squares of fp16 values are exact in fp32), added as
//        a binary tree: relative error at most log2(H) * 2^-24
//   r  = 1 / sqrt(ss / H + eps)   (IEEE division, square root, division;
//        r = 0 when ss / H + eps == 0)
//   y  = fp16((x * r) * w)
// so y is within one fp16 unit in the last place of the correctly rounded
// value, and equal to it except where the exact value lies within a few
// fp32 ulps of a point halfway between two fp16 numbers.  The tree follows
// the thread layout: chunk c (8 values, itself summed as a 3-level tree)
// belongs to thread c % T in slot c / T; lanes then add by xor-shuffles
// (aligned blocks of 2, 4, .., 64 lanes), waves pairwise through LDS, and
// finally the MAXC slots pairwise.  T and MAXC are powers of two with
// T * MAXC chunks >= the row.  Any order would do; a tree keeps the error
// bound logarithmic in H and every step free of atomics.
// ---------------------------------------------------------------------------

// Sum over a wave's lanes as a balanced binary tree over lane index: after
// the step with offset o every lane holds the sum of its aligned block of 2o
// lanes (fp32 addition is commutative, so both lanes of a pair agree).
__device__ __forceinline__ float wave_tree_sum(float v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = v + __shfl_xor(v, o, kWave);
  return v;
}

// Pairwise tree over n (a power of two) consecutive values, in place; returns a[0].
template <int N>
__device__ __forceinline__ float tree_sum(float (&a)[N]) {
#pragma unroll
  for (int s = 1; s < N; s <<= 1)
#pragma unroll
    for (int j = 0; j + s < N; j += 2 * s) a[j] = a[j] + a[j + s];
  return a[0];
}

// Squares of 8 fp16 values summed as ((e0+e1)+(e2+e3))+((e4+e5)+(e6+e7)).
__device__ __forceinline__ float sumsq8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float e[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = half_bits_to_float(w[i] & 0xFFFFu), b = half_bits_to_float(w[i] >> 16);
    e[2 * i] = a * a;
    e[2 * i + 1] = b * b;
  }
  return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

// fp16((x * r) * w) for 8 values: the product rounded to fp32, then to fp16.
// The empty asm makes the fp32 product a value of its own: otherwise the
// compiler fuses the second product and the conversion into one
// mixed-precision multiply that rounds once, straight to fp16, which
// differs from the two roundings where the fp32 product is a tie.
__device__ __forceinline__ uint4 norm8(uint4 xv, uint4 wv, float r) {
  const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, ws[4] = {wv.x, wv.y, wv.z, wv.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = (half_bits_to_float(xs[i] & 0xFFFFu) * r) * half_bits_to_float(ws[i] & 0xFFFFu);
    float hi = (half_bits_to_float(xs[i] >> 16) * r) * half_bits_to_float(ws[i] >> 16);
    asm volatile("" : "+v"(lo), "+v"(hi));
    o[i] = (uint32_t)float_to_half_bits(lo) | ((uint32_t)float_to_half_bits(hi) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int T, int MAXC>
__global__ __launch_bounds__(T) void rmsnorm_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx, int H,
                                                          const uint16_t* __restrict__ w, float eps,
                                                          uint16_t* __restrict__ y, int8_t* __restrict__ q,
                                                          int64_t ldq, int8_t* __restrict__ qfrag,
                                                          float* __restrict__ scale) {
  constexpr int NWV = T / kWave;
  const int t = (int)threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  const int64_t m = blockIdx.x;
  const uint16_t* row = x + m * ldx;
  const int nch = H >> 3;

  uint4 xv[MAXC], wvec[MAXC];
  float part[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + T * i;
    if (c < nch) {
      xv[i] = *reinterpret_cast<const uint4*>(row + 8 * c);
      wvec[i] = *reinterpret_cast<const uint4*>(w + 8 * c);
      part[i] = sumsq8(xv[i]);
    } else {
      xv[i] = wvec[i] = make_uint4(0, 0, 0, 0);
      part[i] = 0.0f;
    }
  }

  // slot i over the T threads: lanes, then waves; then the slots
  __shared__ float wsum[MAXC][NWV];
  __shared__ float wmax[NWV];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const float v = wave_tree_sum(part[i]);
    if (lane == 0) wsum[i][wv] = v;
  }
  __syncthreads();
  float slot[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    float a[NWV];
#pragma unroll
    for (int j = 0; j < NWV; ++j) a[j] = wsum[i][j];
    slot[i] = tree_sum(a);
  }
  const float ss = tree_sum(slot);
  const float tt = ss / (float)H + eps;                 // IEEE division, then add
  const float r = tt > 0.0f ? 1.0f / sqrtf(tt) : 0.0f;  // IEEE square root and division

  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + T * i;
    if (c < nch) {
      xv[i] = norm8(xv[i], wvec[i], r);                 // xv now holds y
      if (y) *reinterpret_cast<uint4*>(y + m * (int64_t)H + 8 * c) = xv[i];
      amax = max(amax, absmax_bits8(xv[i]));
    }
  }
  float a = wave_max(half_bits_to_float(amax));
  if (NWV > 1) {
    if (lane == 0) wmax[wv] = a;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NWV; ++j) a = fmaxf(a, wmax[j]);
  }

  const float s = a / 127.0f;   // as act_quant_kernel
  const float rs = 1.0f / s;
  if (t == 0) scale[m] = a > 0.0f ? s : 0.0f;
  const int G = H / kGroup;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + T * i;
    if (c < nch) put_codes(q, ldq, qfrag, m, G, c, a > 0.0f ? quant8(xv[i], s, rs) : make_uint2(0, 0));
  }
}

}  // namespace

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* w, int64_t M, int64_t H, int64_t ldx, float eps,
                                uint16_t* y, int8_t* q, int64_t ldq, int8_t* qfrag, float* scale, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int64_t nch = H / 8;
  int64_t p = 1;
  while (p < nch) p *= 2;                         // chunks of the padded row
  const dim3 grid((unsigned)M);
  const int64_t threads = std::min<int64_t>(1024, std::max<int64_t>(64, p));
  const int64_t maxc = std::max<int64_t>(1, p / threads);
#define QG_RMS(TH, MC) rmsnorm_quant_kernel<TH, MC><<<grid, dim3(TH), 0, st>>>(x, ldx, (int)H, w, eps, y, q, ldq, qfrag, scale)
  switch (threads * 16 + maxc) {
    case 64 * 16 + 1: QG_RMS(64, 1); break;
    case 128 * 16 + 1: QG_RMS(128, 1); break;
    case 256 * 16 + 1: QG_RMS(256, 1); break;
    case 512 * 16 + 1: QG_RMS(512, 1); break;
    case 1024 * 16 + 1: QG_RMS(1024, 1); break;
    case 1024 * 16 + 2: QG_RMS(1024, 2); break;
    case 1024 * 16 + 4: QG_RMS(1024, 4); break;
    case 1024 * 16 + 8: QG_RMS(1024, 8); break;
    default: return hipErrorInvalidValue;         // rows longer than 65536 (rejected on the host)
  }
#undef QG_RMS
  return hipGetLastError();
}

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
