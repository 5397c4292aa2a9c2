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
// activation codes (128 x 128 B, rows padded to 144 B so 16-byte LDS reads of
// 16 consecutive rows hit distinct banks), the packed int4 weights (8 n-tiles
// x 1 KiB, already in lane order) and the 128 group scales in LDS, double
// buffered: the next group's buffer loads are issued before the current
// group's matrix-core work and written to the other buffer after it.
//
// Rescale.  Per group and tile two v_mfma_i32_16x16x64_i8 give 16 * P
// exactly; acc += fp32(16 P) * s (fp16 scale operand of v_fma_mix), and the
// factor 1/16 joins the token scale in the epilogue.  That is two VALU
// operations per output element per group, as much issue time as the
// matrix-core work itself, so the two are software-pipelined: the 16 tiles
// are split into two halves, and while one half's MFMAs run, the VALU
// rescales the other half's previous partials.
//
// Placement.  Workgroups are dealt to the 8 XCDs round-robin; ids are
// remapped so each XCD walks a contiguous run of a grouped tile order (8
// m-blocks by the n-blocks), and the workgroups resident together on an XCD
// share activation and weight slices in its L2.
#include "common.h"

namespace qg {
namespace {

constexpr int BM = 128, BN = 128, ASTR = 144, GROUP_M = 8;
constexpr uint32_t kHiNib = 0xF0F0F0F0u;
constexpr uint32_t kOOB = 0x80000000u;

struct LargeParams {
  const int8_t* codes;
  const float* tok_scale;
  const uint8_t* w;
  const uint16_t* s;
  int M, N, K, G;
  int mblocks, nblocks, per_xcd;
  uint16_t* y;
  int32_t* dbg;
  int dm0, dm1, dn0, dn1;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// voff: per-lane offset (fixed across the K loop); soff: wave-uniform offset
// of the current group (kept in a scalar register).
__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// acc[t] += fp32(P[t]) * scale, for the 8 tiles t of one half.
__device__ __forceinline__ void rescale_half(f32x4 (&acc)[4][4], const i32x4 (&P)[8], const uint2 (&sc)[4], int h) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int j = 2 * h + t / 4, mt = t % 4;
    const _Float16 s4[4] = {__builtin_bit_cast(_Float16, (uint16_t)(sc[j].x & 0xFFFFu)),
                            __builtin_bit_cast(_Float16, (uint16_t)(sc[j].x >> 16)),
                            __builtin_bit_cast(_Float16, (uint16_t)(sc[j].y & 0xFFFFu)),
                            __builtin_bit_cast(_Float16, (uint16_t)(sc[j].y >> 16))};
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][mt][r] = __builtin_fmaf((float)P[t][r], (float)s4[r], acc[j][mt][r]);
  }
}

template <bool DEBUG>
__global__ __launch_bounds__(256, 2) void w4a8_large_kernel(LargeParams p) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * ASTR];
  __shared__ __attribute__((aligned(16))) uint4 Bs[2][8 * 64];
  // group scales: words 0..63 hold the 128 fp16 scales; every thread stores
  // one word so the store needs no branch (words 64..255 take the zeros of
  // out-of-range loads)
  __shared__ __attribute__((aligned(16))) uint32_t Ss[2][256];

  // Tile of this workgroup (see "Placement").
  const int xcd = blockIdx.x & 7;
  const int t = xcd * p.per_xcd + (int)(blockIdx.x >> 3);
  if (t >= p.mblocks * p.nblocks) return;
  const int per_group = GROUP_M * p.nblocks;
  const int first_m = (t / per_group) * GROUP_M;
  const int gm = min(GROUP_M, p.mblocks - first_m);
  const int mb = first_m + (t % per_group) % gm;
  const int nb = (t % per_group) / gm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int col = lane & 15, quad = lane >> 4;
  const int m0 = mb * BM;
  const int nt_base = nb * 8;
  const int ntiles = p.N / 16;
  const int G = p.G;
  const int mrows = min(BM, p.M - m0);
  const int nvt = min(8, ntiles - nt_base);

  // Range-checked resources: rows past M, n-tiles past N and the prefetch
  // past the last group read zeros without touching memory.
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.codes + (int64_t)m0 * p.K, (uint32_t)(mrows * (int64_t)p.K));
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(p.w + (int64_t)nt_base * G * 1024, (uint32_t)(nvt * (int64_t)G * 1024));
  const __amdgpu_buffer_rsrc_t rsS = make_rsrc(p.s + (int64_t)nt_base * G * 16, (uint32_t)(nvt * (int64_t)G * 32));

  // Per-lane offsets of the staging loads (the group adds a scalar offset).
  uint32_t va[4], vb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    va[i] = (uint32_t)(c >> 3) * (uint32_t)p.K + 16u * (c & 7);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    vb[i] = ((uint32_t)(idx >> 6) * G * 64u + (idx & 63)) * 16u;
  }
  // scales of the 8 n-tiles: thread t < 64 loads rows 2(t&7), +1 of n-tile t>>3
  const uint32_t vs = tid < 64 ? (((uint32_t)(tid >> 3) * G) * 16u + 2u * (tid & 7)) * 2u : kOOB;

  uint4 ra[4], rb[2];
  uint32_t rs;
  auto gload = [&](int g, bool valid) {
    const uint32_t sa = valid ? (uint32_t)g * kGroup : kOOB;
    const uint32_t sb = valid ? (uint32_t)g * 1024u : kOOB;
    const uint32_t ss = valid ? (uint32_t)g * 32u : kOOB;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ld128(rsA, va[i], sa);
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = ld128(rsB, vb[i], sb);
    rs = __builtin_amdgcn_raw_buffer_load_b32(rsS, vs, ss, 0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3, part = c & 7;
      *reinterpret_cast<uint4*>(&As[buf][r * ASTR + 16 * part]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) Bs[buf][tid + 256 * i] = rb[i];
    Ss[buf][tid] = rs;
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[j][mt] = (f32x4)0.0f;

  gload(0, true);
  sstore(0);
  __syncthreads();

  i32x4 P[2][8];     // partials of the two halves of the wave's 16 tiles
  uint2 sc[4], sc_prev[4];
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    gload(g + 1, g + 1 < G);

    i32x4 wa[4][2], xb[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 w = Bs[buf][(wn * 4 + j) * 64 + lane];
      wa[j][0][0] = (int32_t)((w.x << 4) & kHiNib); wa[j][0][1] = (int32_t)(w.x & kHiNib);
      wa[j][0][2] = (int32_t)((w.y << 4) & kHiNib); wa[j][0][3] = (int32_t)(w.y & kHiNib);
      wa[j][1][0] = (int32_t)((w.z << 4) & kHiNib); wa[j][1][1] = (int32_t)(w.z & kHiNib);
      wa[j][1][2] = (int32_t)((w.w << 4) & kHiNib); wa[j][1][3] = (int32_t)(w.w & kHiNib);
      sc[j] = *reinterpret_cast<const uint2*>(&Ss[buf][(wn * 4 + j) * 8 + 2 * quad]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int8_t* src = &As[buf][(wm * 64 + mt * 16 + col) * ASTR + 16 * quad];
      xb[mt][0] = *reinterpret_cast<const i32x4*>(src);
      xb[mt][1] = *reinterpret_cast<const i32x4*>(src + 64);
    }

    // Half 0's MFMAs run beside the rescale of the previous group's half 1,
    // half 1's beside the rescale of half 0 (the rescale of a half never
    // waits for the matrix cores still working on the other half).
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int j = 2 * h + tt / 4, mt = tt % 4;
        i32x4 v = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[j][0], xb[mt][0], (i32x4)0, 0, 0, 0);
        P[h][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[j][1], xb[mt][1], v, 0, 0, 0);
      }
      if (h == 0) {
        if (g > 0) rescale_half(acc, P[1], sc_prev, 1);
      } else {
        rescale_half(acc, P[0], sc, 0);
      }
    }
    if constexpr (DEBUG) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const int j = 2 * h + tt / 4, mt = tt % 4;
          const int m = m0 + wm * 64 + mt * 16 + col;
          if (m >= p.dm0 && m < p.dm1 && m < p.M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int n = (nt_base + wn * 4 + j) * 16 + 4 * quad + r;
              if (n >= p.dn0 && n < p.dn1 && n < p.N)
                p.dbg[((int64_t)(m - p.dm0) * (p.dn1 - p.dn0) + (n - p.dn0)) * G + g] = P[h][tt][r] >> 4;
            }
          }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) sc_prev[j] = sc[j];

    sstore(buf ^ 1);
    __syncthreads();
  }
  if (G > 0) rescale_half(acc, P[1], sc_prev, 1);

#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = m0 + wm * 64 + mt * 16 + col;
    if (m >= p.M) continue;
    const float ts = p.tok_scale[m] * 0.0625f;   // token scale and the 1/16 of the 16*q weights
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
  p.w = reinterpret_cast<const uint8_t*>(a.w);
  p.s = a.s;
  p.M = (int)a.M;
  p.N = (int)a.N;
  p.K = (int)a.K;
  p.G = (int)(a.K / kGroup);
  p.mblocks = (p.M + BM - 1) / BM;
  p.nblocks = (p.N + BN - 1) / BN;
  p.per_xcd = (p.mblocks * p.nblocks + 7) / 8;
  p.y = a.y;
  p.dbg = a.dbg;
  p.dm0 = (int)a.dm0; p.dm1 = (int)a.dm1; p.dn0 = (int)a.dn0; p.dn1 = (int)a.dn1;
  const unsigned grid = (unsigned)(8 * p.per_xcd);
  if (a.dbg)
    w4a8_large_kernel<true><<<grid, 256, 0, st>>>(p);
  else
    w4a8_large_kernel<false><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace qg
