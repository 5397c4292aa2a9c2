// W4A8 GEMM for large token counts (prefill chunks).
//
// "What this repo does that stock vLLM doesn't", section "int8 prefill for
// single-user mode": prefill is compute-bound at every batch size, so the
// W4A8 path (int8 activations, int4 weights, int8 matrix units) is the one
// that pays; "In full" item 4 gives the arithmetic (int32 accumulation per
// 128-wide group, signed group scales).
//
// Tiling.  A workgroup of 4 wavefronts computes a 128 (m) x 128 (n) output
// tile over all K; each wave owns a 64 x 64 quarter = 4 x 4 matrix-core
// tiles of 16 x 16.  Per 128-wide group the workgroup stages the int8
// activation codes (128 x 128 B, rows padded to 144 B so the 16-byte LDS
// reads of 16 consecutive rows hit distinct banks) and the packed int4
// weights (8 n-tiles x 1 KiB, already in lane order) in LDS, double
// buffered: the next group's global loads are issued before the current
// group's matrix-core work and written to the other buffer after it.
// Per group and tile: two v_mfma_i32_16x16x64_i8 give 16 * P exactly, then
// acc += fp32(16 P) * (s_w / 16); the token scale multiplies at the end.
#include "common.h"

namespace qg {
namespace {

constexpr int BM = 128, BN = 128, ASTR = 144;
constexpr uint32_t kHiNib = 0xF0F0F0F0u;

struct LargeParams {
  const int8_t* codes;
  const float* tok_scale;
  const uint4* w;
  const uint16_t* s;
  int M, N, K, G;
  uint16_t* y;
  int32_t* dbg;
  int dm0, dm1, dn0, dn1;
};

template <bool DEBUG>
__global__ __launch_bounds__(256, 2) void w4a8_large_kernel(LargeParams p) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * ASTR];
  __shared__ __attribute__((aligned(16))) uint4 Bs[2][8 * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int col = lane & 15, quad = lane >> 4;
  const int nbn = (p.N + BN - 1) / BN;
  const int mb = blockIdx.x / nbn, nb = blockIdx.x % nbn;
  const int m0 = mb * BM;
  const int nt_base = nb * 8;
  const int ntiles = p.N / 16;
  const int G = p.G;

  uint4 ra[4], rb[2];
  auto gload = [&](int g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3, part = c & 7;
      const int m = m0 + r;
      ra[i] = m < p.M ? *reinterpret_cast<const uint4*>(p.codes + (int64_t)m * p.K + g * kGroup + 16 * part)
                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i, nt = nt_base + (idx >> 6);
      rb[i] = nt < ntiles ? p.w[((int64_t)nt * G + g) * 64 + (idx & 63)] : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3, part = c & 7;
      *reinterpret_cast<uint4*>(&As[buf][r * ASTR + 16 * part]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) Bs[buf][tid + 256 * i] = rb[i];
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[j][mt] = (f32x4)0.0f;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const bool more = g + 1 < G;
    if (more) gload(g + 1);

    float sc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nt = nt_base + wn * 4 + j;
      const uint2 sv = nt < ntiles ? *reinterpret_cast<const uint2*>(p.s + ((int64_t)nt * G + g) * 16 + 4 * quad)
                                   : make_uint2(0, 0);
      sc[j][0] = half_bits_to_float(sv.x & 0xFFFFu) * 0.0625f;
      sc[j][1] = half_bits_to_float(sv.x >> 16) * 0.0625f;
      sc[j][2] = half_bits_to_float(sv.y & 0xFFFFu) * 0.0625f;
      sc[j][3] = half_bits_to_float(sv.y >> 16) * 0.0625f;
    }

    i32x4 xb[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int8_t* src = &As[buf][(wm * 64 + mt * 16 + col) * ASTR + 16 * quad];
      xb[mt][0] = *reinterpret_cast<const i32x4*>(src);
      xb[mt][1] = *reinterpret_cast<const i32x4*>(src + 64);
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 w = Bs[buf][(wn * 4 + j) * 64 + lane];
      i32x4 a0, a1;
      a0[0] = (int32_t)((w.x << 4) & kHiNib); a0[1] = (int32_t)(w.x & kHiNib);
      a0[2] = (int32_t)((w.y << 4) & kHiNib); a0[3] = (int32_t)(w.y & kHiNib);
      a1[0] = (int32_t)((w.z << 4) & kHiNib); a1[1] = (int32_t)(w.z & kHiNib);
      a1[2] = (int32_t)((w.w << 4) & kHiNib); a1[3] = (int32_t)(w.w & kHiNib);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        i32x4 P = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, xb[mt][0], (i32x4)0, 0, 0, 0);
        P = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, xb[mt][1], P, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][mt][r] = fmaf((float)P[r], sc[j][r], acc[j][mt][r]);
        if constexpr (DEBUG) {
          const int m = m0 + wm * 64 + mt * 16 + col;
          if (m >= p.dm0 && m < p.dm1 && m < p.M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int n = (nt_base + wn * 4 + j) * 16 + 4 * quad + r;
              if (n >= p.dn0 && n < p.dn1 && n < p.N)
                p.dbg[((int64_t)(m - p.dm0) * (p.dn1 - p.dn0) + (n - p.dn0)) * G + g] = P[r] >> 4;
            }
          }
        }
      }
    }

    if (more) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = m0 + wm * 64 + mt * 16 + col;
    if (m >= p.M) continue;
    const float ts = p.tok_scale[m];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nt = nt_base + wn * 4 + j;
      if (nt >= ntiles) continue;
      const int n = nt * 16 + 4 * quad;
      uint2 o;
      o.x = (uint32_t)float_to_half_bits(acc[j][mt][0] * ts) | ((uint32_t)float_to_half_bits(acc[j][mt][1] * ts) << 16);
      o.y = (uint32_t)float_to_half_bits(acc[j][mt][2] * ts) | ((uint32_t)float_to_half_bits(acc[j][mt][3] * ts) << 16);
      *reinterpret_cast<uint2*>(p.y + (int64_t)m * p.N + n) = o;
    }
  }
}

}  // namespace

hipError_t launch_w4a8_large(const LargeArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  LargeParams p;
  p.codes = a.codes;
  p.tok_scale = a.tok_scale;
  p.w = reinterpret_cast<const uint4*>(a.w);
  p.s = a.s;
  p.M = (int)a.M;
  p.N = (int)a.N;
  p.K = (int)a.K;
  p.G = (int)(a.K / kGroup);
  p.y = a.y;
  p.dbg = a.dbg;
  p.dm0 = (int)a.dm0; p.dm1 = (int)a.dm1; p.dn0 = (int)a.dn0; p.dn1 = (int)a.dn1;
  const unsigned grid = (unsigned)(((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN));
  if (a.dbg)
    w4a8_large_kernel<true><<<grid, 256, 0, st>>>(p);
  else
    w4a8_large_kernel<false><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace qg
