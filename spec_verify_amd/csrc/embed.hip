// int8 group-128 vocabulary table: dequant-on-gather lookup and the offline
// requantisation from bf16.
//
// "What this repo does that stock vLLM doesn't", "In full" item 1: lm_head
// and embed_tokens are requantised from bf16 to int8 group-128 (about 0.6%
// round-trip error); item 2: a dequant-on-gather kernel serves the int8
// embedding table.  Both kernels here are bit-exact: the gather's fp32
// product int8 * fp16 is exact and is rounded once to fp16; the
// requantisation uses IEEE fp32 division and round-half-to-even.
#include "common.h"

namespace qg {
namespace {

// One thread converts 8 consecutive values of one row (8 bytes in, 16 out).
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                     const int8_t* __restrict__ table,
                                                     const uint16_t* __restrict__ scales, int64_t V,
                                                     int H, uint16_t* __restrict__ out) {
  const int per_row = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row;
  const int c = (int)(idx % per_row);
  const int32_t id = ids[t];
  uint4 o = make_uint4(0, 0, 0, 0);
  if (id >= 0 && id < V) {
    const uint2 q = *reinterpret_cast<const uint2*>(table + (int64_t)id * H + 8 * c);
    const float s = half_bits_to_float(scales[(int64_t)id * (H / kGroup) + (8 * c) / kGroup]);
    const uint32_t b[2] = {q.x, q.y};
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = b[i >> 1] >> (16 * (i & 1));
      const float v0 = (float)(int8_t)(w & 0xFFu) * s;
      const float v1 = (float)(int8_t)((w >> 8) & 0xFFu) * s;
      h[i] = (uint32_t)float_to_half_bits(v0) | ((uint32_t)float_to_half_bits(v1) << 16);
    }
    o = make_uint4(h[0], h[1], h[2], h[3]);
  }
  *reinterpret_cast<uint4*>(out + t * H + 8 * c) = o;
}

// One wavefront per 128-value group: each lane owns 2 adjacent values.
__global__ __launch_bounds__(256) void quant_table_kernel(const uint16_t* __restrict__ src, int64_t ngroups,
                                                          int8_t* __restrict__ Q, uint16_t* __restrict__ S) {
  const int lane = threadIdx.x & 63;
  const int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp >= ngroups) return;
  const uint32_t pair = *reinterpret_cast<const uint32_t*>(src + grp * kGroup + 2 * lane);
  const float v0 = __builtin_bit_cast(float, pair << 16);
  const float v1 = __builtin_bit_cast(float, pair & 0xFFFF0000u);
  const float a = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const uint16_t sb = float_to_half_bits(a / 127.0f);      // fp16(fp32(a) / 127)
  const float sf = half_bits_to_float(sb);
  int q0 = 0, q1 = 0;
  if (sf != 0.0f) {
    q0 = (int)fminf(fmaxf(rintf(v0 / sf), -127.0f), 127.0f);
    q1 = (int)fminf(fmaxf(rintf(v1 / sf), -127.0f), 127.0f);
  }
  *reinterpret_cast<uint16_t*>(Q + grp * kGroup + 2 * lane) = (uint16_t)((q0 & 0xFF) | ((q1 & 0xFF) << 8));
  if (lane == 0) S[grp] = sb;
}

}  // namespace

hipError_t launch_gather(const int32_t* ids, int64_t T, const int8_t* table, const uint16_t* scales,
                         int64_t V, int64_t H, uint16_t* out, hipStream_t st) {
  const int64_t total = T * (H / 8);
  if (total == 0) return hipSuccess;
  gather_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(ids, T, table, scales, V, (int)H, out);
  return hipGetLastError();
}

hipError_t launch_quant_table(const uint16_t* src, int64_t V, int64_t H, int8_t* Q, uint16_t* S,
                              hipStream_t st) {
  const int64_t ngroups = V * (H / kGroup);
  if (ngroups == 0) return hipSuccess;
  quant_table_kernel<<<(unsigned)((ngroups + 3) / 4), 256, 0, st>>>(src, ngroups, Q, S);
  return hipGetLastError();
}

}  // namespace qg
