// Load-time repack of canonical int4 weights into the layout the GEMMs stream.
//
// Canonical input ("What this repo does that stock vLLM doesn't", "In full"
// item 4): codes[N][K] in [-8, 7] and signed fp16 scales[N][K/128].  Signs
// stay where they are: a fold of the scale's sign into the codes cannot
// represent -(-8) = +8 in int4, so the kernels apply signed scales directly.
//
// Packed layout.  Weights are cut into blocks of 16 rows (an "n-tile") by
// one 128-wide group; block (nt, g) is 1 KiB at byte offset
// ((nt * G) + g) * 1024, n-tile major, so one n-tile's groups are contiguous.
// Inside a block, lane l of a wavefront owns the 16 bytes at l * 16:
//   row  n  = 16 * nt + (l % 16),  quarter kb = l / 16,
//   word i (i = 0..3) covers k = 128 g + 64 (i / 2) + 16 kb + 8 (i % 2) + [0, 8),
//   nibble slot s (bits 4s..4s+3) of a word holds k offset (s % 2) * 4 + s / 2.
// With that slot order, (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0 give the
// int8 values 16*q for k offsets 0..3 and 4..7 in natural byte order, which
// is what the int8 matrix-core operand of one lane needs; words 0-1 feed the
// first 64 k of the group and words 2-3 the second 64.
// Packed scales: for block (nt, g), the 16 fp16 scales of rows 16 nt .. +15
// at element offset ((nt * G) + g) * 16.
#include "common.h"

namespace qg {
namespace {

__global__ __launch_bounds__(256) void w4_repack_kernel(const int8_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scales,
                                                        int64_t N, int K, uint4* __restrict__ wp,
                                                        uint16_t* __restrict__ sp) {
  const int G = K / kGroup;
  const int64_t total = (N / 16) * G * 64;        // one thread per 16-byte lane slot
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  const int64_t blk = idx >> 6;                    // nt * G + g
  const int g = (int)(blk % G);
  const int64_t nt = blk / G;
  const int64_t n = nt * 16 + (lane & 15);
  const int kb = lane >> 4;
  const int8_t* crow = codes + n * K;

  uint32_t words[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k0 = g * kGroup + 64 * (i >> 1) + 16 * kb + 8 * (i & 1);
    const uint2 raw = *reinterpret_cast<const uint2*>(crow + k0);   // codes k0 .. k0+7
    const uint32_t b[2] = {raw.x, raw.y};
    uint32_t w = 0;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int off = (s & 1) * 4 + (s >> 1);
      const uint32_t code = (b[off >> 2] >> (8 * (off & 3))) & 0xFu;
      w |= code << (4 * s);
    }
    words[i] = w;
  }
  wp[idx] = make_uint4(words[0], words[1], words[2], words[3]);
  if (kb == 0) sp[blk * 16 + (lane & 15)] = scales[n * G + g];
}

}  // namespace

hipError_t launch_w4_repack(const int8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                            void* w_packed, uint16_t* s_packed, hipStream_t st) {
  const int64_t total = (N / 16) * (K / kGroup) * 64;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  w4_repack_kernel<<<blocks, 256, 0, st>>>(codes, scales, N, (int)K,
                                           reinterpret_cast<uint4*>(w_packed), s_packed);
  return hipGetLastError();
}

}  // namespace qg
