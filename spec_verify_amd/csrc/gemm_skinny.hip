// Weight-streaming GEMMs for small token counts (M <= 64): batched decode,
// speculative verify (M = 1 + draft tokens) and the int8 lm_head.
//
// Sources: "What this repo does that stock vLLM doesn't", "In full" items 4
// (W4A8: int8 activations x int4 weights, int32 accumulation per group,
// signed group scales) and 5 (the int8 lm_head read per draft); the project
// README, "What each step buys" (W4A16 body).  At these M the product reads
// each weight byte once and does little arithmetic per byte, so the kernel is
// built to keep HBM busy: every wavefront streams 1 KiB weight blocks with
// 128-bit loads, one group ahead of the matrix-core work.
//
// Work split.  A workgroup (4 wavefronts) owns 64 output columns (4 n-tiles
// of 16 rows of W) and a contiguous range of K groups ("split"); its waves
// take that range's groups round-robin, so every activation byte is read once
// per workgroup.  The four waves' fp32 sums are added in LDS in a fixed
// order; with more than one split, each split writes fp32 partial sums and a
// second kernel adds the splits in index order.  No floating-point atomics:
// results are bit-reproducible.
//
// Matrix-core mapping.  Weights are the A operand (rows n), activations the B
// operand (columns m), so a 16x16 output tile lands as 4 consecutive n for
// one m in each lane.  Per 128-wide group:
//   W4A8   2 x v_mfma_i32_16x16x64_i8 on (16*q_w, q_a) -> 16*P exactly, then
//          acc += fp32(16*P) * (s_w / 16)      (exact scaling by 1/16)
//   W4A16  4 x v_mfma_f32_16x16x32_f16 on exact fp16 codes q_w and fp16 x,
//          then acc += group_sum * s_w
//   W8A16  as W4A16 with int8 table codes converted exactly to fp16.
// The k order inside a lane operand is a permutation shared by both operands,
// so the contraction is unaffected by it.
#include "common.h"

namespace qg {
namespace {

struct SkinnyParams {
  const void* act;
  int64_t lda;
  const float* tok_scale;
  const void* w;
  const uint16_t* s;
  int M, N, K, G;
  int splits, gps;          // number of K splits, groups per split
  uint16_t* y;
  float* partials;
  int32_t* dbg;
  int dm0, dm1, dn0, dn1;
};

constexpr uint32_t kHiNib = 0xF0F0F0F0u;

// int8 operand (16 values 16*q) from two packed words; see repack.hip for the
// nibble order that makes this the natural k order.
__device__ __forceinline__ i32x4 w4_to_i8x16(uint32_t w0, uint32_t w1) {
  i32x4 r;
  r[0] = (int32_t)((w0 << 4) & kHiNib);
  r[1] = (int32_t)(w0 & kHiNib);
  r[2] = (int32_t)((w1 << 4) & kHiNib);
  r[3] = (int32_t)(w1 & kHiNib);
  return r;
}

// Exact fp16 values of the 8 int4 codes of one packed word:
// 0x6400 | (nibble ^ 8) is the fp16 number 1024 + q + 8.  Element order is
// k offsets {0, 2, 4, 6, 1, 3, 5, 7} (see kW4A16 activation shuffle).
__device__ __forceinline__ f16x8 w4_to_f16x8(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  u32x4 p;
  p[0] = (x & 0x000F000Fu) | 0x64006400u;
  p[1] = ((x >> 4) & 0x000F000Fu) | 0x64006400u;
  p[2] = ((x >> 8) & 0x000F000Fu) | 0x64006400u;
  p[3] = ((x >> 12) & 0x000F000Fu) | 0x64006400u;
  return __builtin_bit_cast(f16x8, p) - (f16x8)(_Float16)1032.0f;
}

// Exact fp16 values of 8 int8 codes (natural order): byte b ^ 0x80 = b + 128
// placed under exponent byte 0x64 is 1024 + b + 128.
__device__ __forceinline__ f16x8 i8_to_f16x8(uint32_t w0, uint32_t w1) {
  const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
  u32x4 p;
  p[0] = __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u);
  p[1] = __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u);
  p[2] = __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u);
  p[3] = __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u);
  return __builtin_bit_cast(f16x8, p) - (f16x8)(_Float16)1152.0f;
}

template <int MODE, int MT>
struct Stage;

template <int MT>
struct Stage<kW4A8, MT> {
  uint4 w[4];
  uint2 s[4];
  i32x4 x[MT][2];
};

template <int MT>
struct Stage<kW4A16, MT> {
  uint4 w[4];
  uint2 s[4];
  f16x8 x[MT][4];
};

template <int MT>
struct Stage<kW8A16, MT> {
  uint4 w[4][2];
  uint16_t s[4][4];
  f16x8 x[MT][4];
};

template <int MODE, int MT>
__device__ __forceinline__ void load_stage(const SkinnyParams& p, Stage<MODE, MT>& st, int g, int nt0,
                                           int nvalid, int lane) {
  const int col = lane & 15, quad = lane >> 4;
  const int G = p.G;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < nvalid) {
      const int64_t blk = (int64_t)(nt0 + j) * G + g;
      if constexpr (MODE == kW8A16) {
        const int8_t* row = reinterpret_cast<const int8_t*>(p.w) +
                            ((int64_t)(nt0 + j) * 16 + col) * p.K + g * kGroup + 16 * quad;
        st.w[j][0] = *reinterpret_cast<const uint4*>(row);
        st.w[j][1] = *reinterpret_cast<const uint4*>(row + 64);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st.s[j][r] = p.s[((int64_t)(nt0 + j) * 16 + 4 * quad + r) * G + g];
      } else {
        st.w[j] = reinterpret_cast<const uint4*>(p.w)[blk * 64 + lane];
        st.s[j] = *reinterpret_cast<const uint2*>(p.s + blk * 16 + 4 * quad);
      }
    } else {
      if constexpr (MODE == kW8A16) {
        st.w[j][0] = st.w[j][1] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) st.s[j][r] = 0;
      } else {
        st.w[j] = make_uint4(0, 0, 0, 0);
        st.s[j] = make_uint2(0, 0);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + col;
    if constexpr (MODE == kW4A8) {
      if (m < p.M) {
        const int8_t* src = reinterpret_cast<const int8_t*>(p.act) + (int64_t)m * p.lda + g * kGroup + 16 * quad;
        st.x[mt][0] = *reinterpret_cast<const i32x4*>(src);
        st.x[mt][1] = *reinterpret_cast<const i32x4*>(src + 64);
      } else {
        st.x[mt][0] = st.x[mt][1] = (i32x4)0;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (m < p.M) {
          const uint16_t* src = reinterpret_cast<const uint16_t*>(p.act) + (int64_t)m * p.lda + g * kGroup +
                                64 * (t >> 1) + 16 * quad + 8 * (t & 1);
          const f16x8 v = *reinterpret_cast<const f16x8*>(src);
          if constexpr (MODE == kW4A16)
            st.x[mt][t] = __builtin_shufflevector(v, v, 0, 2, 4, 6, 1, 3, 5, 7);
          else
            st.x[mt][t] = v;
        } else {
          st.x[mt][t] = (f16x8)(_Float16)0.0f;
        }
      }
    }
  }
}

template <int MODE, int MT, bool DEBUG>
__device__ __forceinline__ void compute_stage(const SkinnyParams& p, const Stage<MODE, MT>& st, int g,
                                              int nt0, int nvalid, int lane, f32x4 (&acc)[4][MT]) {
  const int col = lane & 15, quad = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j >= nvalid) continue;
    float sc[4];
    if constexpr (MODE == kW8A16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = half_bits_to_float(st.s[j][r]);
    } else {
      sc[0] = half_bits_to_float(st.s[j].x & 0xFFFFu);
      sc[1] = half_bits_to_float(st.s[j].x >> 16);
      sc[2] = half_bits_to_float(st.s[j].y & 0xFFFFu);
      sc[3] = half_bits_to_float(st.s[j].y >> 16);
    }
    if constexpr (MODE == kW4A8) {
      const i32x4 a0 = w4_to_i8x16(st.w[j].x, st.w[j].y);
      const i32x4 a1 = w4_to_i8x16(st.w[j].z, st.w[j].w);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] *= 0.0625f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        i32x4 P = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.x[mt][0], (i32x4)0, 0, 0, 0);
        P = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.x[mt][1], P, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][mt][r] = fmaf((float)P[r], sc[r], acc[j][mt][r]);
        if constexpr (DEBUG) {
          const int m = mt * 16 + col;
          if (m >= p.dm0 && m < p.dm1 && m < p.M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int n = (nt0 + j) * 16 + 4 * quad + r;
              if (n >= p.dn0 && n < p.dn1)
                p.dbg[((int64_t)(m - p.dm0) * (p.dn1 - p.dn0) + (n - p.dn0)) * p.G + g] = P[r] >> 4;
            }
          }
        }
      }
    } else {
      f16x8 a[4];
      if constexpr (MODE == kW4A16) {
        a[0] = w4_to_f16x8(st.w[j].x);
        a[1] = w4_to_f16x8(st.w[j].y);
        a[2] = w4_to_f16x8(st.w[j].z);
        a[3] = w4_to_f16x8(st.w[j].w);
      } else {
        a[0] = i8_to_f16x8(st.w[j][0].x, st.w[j][0].y);
        a[1] = i8_to_f16x8(st.w[j][0].z, st.w[j][0].w);
        a[2] = i8_to_f16x8(st.w[j][1].x, st.w[j][1].y);
        a[3] = i8_to_f16x8(st.w[j][1].z, st.w[j][1].w);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], st.x[mt][0], (f32x4)0.0f, 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], st.x[mt][1], gs, 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2], st.x[mt][2], gs, 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[3], st.x[mt][3], gs, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][mt][r] = fmaf(gs[r], sc[r], acc[j][mt][r]);
      }
    }
  }
}

template <int MODE, int MT, bool DEBUG>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int split = blockIdx.x % p.splits;
  const int nb = blockIdx.x / p.splits;
  const int g0 = split * p.gps;
  const int g1 = min(p.G, g0 + p.gps);
  const int nt0 = nb * 4;
  const int nvalid = min(4, p.N / 16 - nt0);

  f32x4 acc[4][MT];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x4)0.0f;

  int g = g0 + wave;
  if (g < g1) {
    Stage<MODE, MT> cur;
    load_stage<MODE, MT>(p, cur, g, nt0, nvalid, lane);
    for (; g < g1; g += 4) {
      Stage<MODE, MT> nxt;
      const bool more = g + 4 < g1;
      if (more) load_stage<MODE, MT>(p, nxt, g + 4, nt0, nvalid, lane);
      compute_stage<MODE, MT, DEBUG>(p, cur, g, nt0, nvalid, lane, acc);
      if (more) cur = nxt;
    }
  }

  // Fixed-order sum of the four waves' partial results.
  __shared__ float red[4][4 * MT * 4][64];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][(j * MT + mt) * 4 + r][lane] = acc[j][mt][r];
  __syncthreads();

  for (int idx = threadIdx.x; idx < 4 * MT * 64; idx += 256) {
    const int l = idx & 63, jm = idx >> 6;
    const int j = jm / MT, mt = jm % MT;
    const int m = mt * 16 + (l & 15);
    if (j >= nvalid || m >= p.M) continue;
    const int n = (nt0 + j) * 16 + 4 * (l >> 4);
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = jm * 4 + r;
      v[r] = ((red[0][e][l] + red[1][e][l]) + red[2][e][l]) + red[3][e][l];
    }
    if (p.splits == 1) {
      const float ts = MODE == kW4A8 ? p.tok_scale[m] : 1.0f;
      uint2 o;
      o.x = (uint32_t)float_to_half_bits(v[0] * ts) | ((uint32_t)float_to_half_bits(v[1] * ts) << 16);
      o.y = (uint32_t)float_to_half_bits(v[2] * ts) | ((uint32_t)float_to_half_bits(v[3] * ts) << 16);
      *reinterpret_cast<uint2*>(p.y + (int64_t)m * p.N + n) = o;
    } else {
      *reinterpret_cast<float4*>(p.partials + ((int64_t)split * p.M + m) * p.N + n) =
          make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// y[m][n] = fp16(tok[m] * sum_{s < S} part[s][m][n]), splits added in index order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S, int M,
                                                            int N, const float* __restrict__ tok,
                                                            uint16_t* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)M * (N / 4);
  if (idx >= total) return;
  const int m = (int)(idx / (N / 4));
  const int64_t off = (int64_t)m * N + 4 * (idx % (N / 4));
  float4 a = *reinterpret_cast<const float4*>(part + off);
  for (int s = 1; s < S; ++s) {
    const float4 b = *reinterpret_cast<const float4*>(part + (int64_t)s * M * N + off);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  const float ts = tok ? tok[m] : 1.0f;
  uint2 o;
  o.x = (uint32_t)float_to_half_bits(a.x * ts) | ((uint32_t)float_to_half_bits(a.y * ts) << 16);
  o.y = (uint32_t)float_to_half_bits(a.z * ts) | ((uint32_t)float_to_half_bits(a.w * ts) << 16);
  *reinterpret_cast<uint2*>(y + off) = o;
}

template <int MODE, bool DEBUG>
hipError_t launch_mode(const SkinnyParams& p, int mt, dim3 grid, hipStream_t st) {
  switch (mt) {
    case 1: skinny_kernel<MODE, 1, DEBUG><<<grid, 256, 0, st>>>(p); break;
    case 2: skinny_kernel<MODE, 2, DEBUG><<<grid, 256, 0, st>>>(p); break;
    case 3: skinny_kernel<MODE, 3, DEBUG><<<grid, 256, 0, st>>>(p); break;
    default: skinny_kernel<MODE, 4, DEBUG><<<grid, 256, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace

int skinny_splits(int64_t N, int64_t K) {
  const int64_t nblocks = (N / 16 + 3) / 4;
  const int64_t G = K / kGroup;
  int s = 1;
  // Split K until the grid covers the 256 compute units, keeping at least
  // two groups per wavefront in every split.
  while (nblocks * s < 256 && G / (2 * s) >= 8) s *= 2;
  return s;
}

hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  SkinnyParams p;
  p.act = a.act;
  p.lda = a.lda;
  p.tok_scale = a.tok_scale;
  p.w = a.w;
  p.s = a.s;
  p.M = (int)a.M;
  p.N = (int)a.N;
  p.K = (int)a.K;
  p.G = (int)(a.K / kGroup);
  p.splits = skinny_splits(a.N, a.K);
  p.gps = (p.G + p.splits - 1) / p.splits;
  p.y = a.y;
  p.partials = a.partials;
  p.dbg = a.dbg;
  p.dm0 = (int)a.dm0; p.dm1 = (int)a.dm1; p.dn0 = (int)a.dn0; p.dn1 = (int)a.dn1;
  const int nblocks = (p.N / 16 + 3) / 4;
  const dim3 grid((unsigned)(nblocks * p.splits));
  const int mt = (p.M + 15) / 16;
  hipError_t e;
  switch (a.mode) {
    case kW4A8:
      e = a.dbg ? launch_mode<kW4A8, true>(p, mt, grid, st) : launch_mode<kW4A8, false>(p, mt, grid, st);
      break;
    case kW4A16: e = launch_mode<kW4A16, false>(p, mt, grid, st); break;
    default: e = launch_mode<kW8A16, false>(p, mt, grid, st); break;
  }
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t total = (int64_t)p.M * (p.N / 4);
  splitk_reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(
      p.partials, p.splits, p.M, p.N, a.mode == kW4A8 ? p.tok_scale : nullptr, p.y);
  return hipGetLastError();
}

}  // namespace qg
