// Split-KV attention for the speculative-verify step: T query tokens (1 + k
// drafts) of one sequence against its KV cache, causal within the block.
//
// Source: "What this repo does that stock vLLM doesn't", "In full" item 6:
// a decode attention that splits the KV sequence across workgroups only when
// a request has one query token leaves most of the GPU idle on a multi-query
// verify step; splitting the KV sequence for the multi-query case fixes it
// (24 query heads, head_dim 256, 1.5k-16k context on the pages).
//
// Definition (fp32 scores and softmax, fp16 output), for query t of T, query
// head h, KV head h / G (G = Hq / Hkv), cache length L (the T verify tokens
// are its last T positions):
//   s(t, h, p) = (q[t][h] . k[p][h/G]) / sqrt(256),  p <= L - T + t
//   o[t][h]    = sum_p softmax_p(s) v[p][h/G]
//
// Pass 1, one workgroup per (split of the cache, KV head): the T*G query rows
// of that KV head (up to 128) against the split's positions, 32 at a time.
// K and V blocks are staged in LDS; scores come out of the matrix cores as
// S^T = K Q^T, so a lane holds 4 positions of one row; the running max, sum
// and output of each row stay in that row's lanes; the product with V is
// O^T = V^T P^T, which takes P straight from the score registers.  Each
// split writes its row maxima, sums and unnormalised outputs (fp32).
// Pass 2 combines the splits per row: o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Scores are kept in log2 units (scaled by log2(e) / 16) so that exp is exp2.
#include <algorithm>

#include "common.h"

namespace qg {
namespace {

constexpr int kD = 256;           // head dimension
constexpr int kBlk = 32;          // positions per staged block
constexpr int kVtStride = 36;     // halves per transposed-V row (32 positions + 4)

// Transposed V in LDS: dimension d's 32 positions form 8 groups of 4
// consecutive positions (8 bytes); group j is stored at slot j ^ ((d / 16) % 8)
// of row d.  The matrix-core reads (16 consecutive dimensions, 4 groups) and
// the staging writes (dimensions 8 apart, one group) then fall in distinct
// bank groups.
__device__ __forceinline__ int vt_at(int d, int group) { return d * kVtStride + 4 * (group ^ ((d >> 4) & 7)); }

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

struct AttnParams {
  const uint16_t* q;      // fp16 [T][Hq][256]
  const uint16_t* k;      // fp16 [L][Hkv][256]
  const uint16_t* v;      // fp16 [L][Hkv][256]
  float* ws_o;            // fp32 [S][Hkv][R][256]
  float* ws_ml;           // fp32 [S][Hkv][R][2]: row max (log2 units), row sum
  uint16_t* o;            // fp16 [T][Hq][256]
  int T, Hq, Hkv, G, R, L, C, S;
};

// K and Q rows in LDS: 32 16-byte pieces per row, piece p of row r stored at
// p ^ (r % 16), so 16 lanes reading the same piece of 16 consecutive rows
// hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int piece) { return row * 32 + (piece ^ (row & 15)); }

// V pieces of 4 consecutive positions (group g of the block) for dims
// 8 piece .. 8 piece + 7, transposed into the LDS layout: one 8-byte store
// per dimension.
__device__ __forceinline__ void stage_v(uint16_t* vt_lds, const uint4* v, int piece, int g) {
  const uint32_t w[4][4] = {{v[0].x, v[0].y, v[0].z, v[0].w},
                            {v[1].x, v[1].y, v[1].z, v[1].w},
                            {v[2].x, v[2].y, v[2].z, v[2].w},
                            {v[3].x, v[3].y, v[3].z, v[3].w}};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int sh = 16 * (e & 1);
    const uint32_t h0 = (w[0][e >> 1] >> sh) & 0xFFFFu, h1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
    const uint32_t h2 = (w[2][e >> 1] >> sh) & 0xFFFFu, h3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
    *reinterpret_cast<uint2*>(&vt_lds[vt_at(8 * piece + e, g)]) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
  }
}

// One 32-position block for one 16-row m-tile of the split: scores from the
// staged K (S^T = K Q^T, a lane holding 4 positions of row mt*16 + col), the
// online softmax update of the row's maximum, sum and output, and
// O^T += V^T P^T from the staged transposed V.
__device__ __forceinline__ void attn_tile_block(const AttnParams& p, const uint4* q_lds, const uint4* k_lds,
                                                const uint16_t* vt_lds, int b0, int p_end, int mt, int col, int quad,
                                                f32x4 (&acc)[16], float& m_run, float& l_run) {
  const float kScale = 1.4426950408889634f / 16.0f;   // log2(e) / sqrt(256)
  constexpr float kLazy = 8.0f;                        // exponentials below 2^8 (fp16 P)
  const int row = mt * 16 + col;
  const int t = row / p.G;
  const int last = p.L - p.T + t;              // last position query t sees
  // scores for the block: two 16-position tiles, lane = (row col, positions 4 quad ..)
  f32x4 s[2];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
    f32x4 c = (f32x4)0.0f;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int piece = 4 * sl + quad;
      const f16x8 a = __builtin_bit_cast(f16x8, k_lds[swz(16 * pt + col, piece)]);
      const f16x8 bq = __builtin_bit_cast(f16x8, q_lds[swz(row, piece)]);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq, c, 0, 0, 0);
    }
    s[pt] = c;
  }
  // The S^T tile has positions in rows (4 quad + j) and query rows in
  // columns (col): lane holds s(row = mt*16 + col, pos = b0 + 16 pt + 4 quad + j).
  float bmax = -__builtin_inff();
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = b0 + 16 * pt + 4 * quad + j;
      const bool ok = row < p.R && pos < p_end && pos <= last;
      s[pt][j] = ok ? s[pt][j] * kScale : -__builtin_inff();
      bmax = fmaxf(bmax, s[pt][j]);
    }
  bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
  bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
  // The reference maximum of a row moves only when some row of the wave
  // sees a block maximum more than kLazy above its own: otherwise the
  // exponentials stay below 2^kLazy and the running output is not
  // rescaled (a row's first finite block always moves it).
  const bool rescale = __ballot(bmax > m_run + kLazy) != 0;   // wave-uniform
  float m_new = m_run, alpha = 1.0f;
  if (rescale) {
    m_new = fmaxf(m_run, bmax);
    alpha = m_new > -__builtin_inff() ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = acc[d] * alpha;
  }
  const bool any = m_new > -__builtin_inff();
  float psum = 0.0f;
  f16x4 pv[2];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = any ? __builtin_amdgcn_exp2f(s[pt][j] - m_new) : 0.0f;
      psum += e;
      pv[pt][j] = (_Float16)e;
    }
  psum += __shfl_xor(psum, 16, 64);
  psum += __shfl_xor(psum, 32, 64);
  l_run = l_run * alpha + psum;
  m_run = m_new;
  // O^T[dim][row] += V^T P^T over the block's two position tiles
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    f32x4 c = acc[d];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const uint2 raw = *reinterpret_cast<const uint2*>(&vt_lds[vt_at(16 * d + col, 4 * pt + quad)]);
      const f16x4 av = __builtin_bit_cast(f16x4, raw);
      c = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pv[pt], c, 0, 0, 0);
    }
    acc[d] = c;
  }
}

template <int MTW>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int col = lane & 15, quad = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int p_begin = split * p.C;
  const int p_end = min(p.L, p_begin + p.C);
  const int MT = (p.R + 15) >> 4;
  const int rowstride = p.Hkv * kD;                    // elements between positions of one KV head

  __shared__ __attribute__((aligned(16))) uint4 q_lds[MTW * 64 * 32];   // up to 64 (MTW 1) or 128 rows
  __shared__ __attribute__((aligned(16))) uint4 k_lds[kBlk * 32];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kD * kVtStride];

  // Q rows of this KV head: row r = t * G + g is query t, head kvh * G + g.
  for (int idx = tid; idx < MT * 16 * 32; idx += 256) {
    const int r = idx >> 5, piece = idx & 31;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < p.R) {
      const int t = r / p.G, h = kvh * p.G + r % p.G;
      val = *reinterpret_cast<const uint4*>(p.q + ((int64_t)t * p.Hq + h) * kD + 8 * piece);
    }
    q_lds[swz(r, piece)] = val;
  }

  // This wave's m-tiles: wave + 4 i.
  f32x4 acc[MTW][16];         // O^T tiles: [m-tile][dim tile], lane = (row col, dims 4 quad ..)
  float m_run[MTW], l_run[MTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    m_run[i] = -__builtin_inff();
    l_run[i] = 0.0f;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[i][d] = (f32x4)0.0f;
  }
  const uint16_t* kbase = p.k + (int64_t)kvh * kD;
  const uint16_t* vbase = p.v + (int64_t)kvh * kD;
  // K and V of a block: thread tid holds the 16-byte piece tid % 32 (dims
  // 8 (tid % 32) ..) of positions 4 (tid / 32) + pass, pass = 0..3, so its
  // four V pieces hold 4 consecutive positions of 8 dimensions.  The next
  // block's are loaded into registers while the current one is multiplied.
  const int kpiece = tid & 31, pgrp = tid >> 5;
  uint4 kreg[4], vreg[4];
  auto fetch = [&](int b0) {
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int pos = b0 + 4 * pgrp + pass;
      kreg[pass] = vreg[pass] = make_uint4(0, 0, 0, 0);
      if (pos < p_end) {
        kreg[pass] = *reinterpret_cast<const uint4*>(kbase + (int64_t)pos * rowstride + 8 * kpiece);
        vreg[pass] = *reinterpret_cast<const uint4*>(vbase + (int64_t)pos * rowstride + 8 * kpiece);
      }
    }
  };
  fetch(p_begin);
  for (int b0 = p_begin; b0 < p_end; b0 += kBlk) {
    __syncthreads();                                   // previous block's LDS reads are done
    // K row-major (swizzled), V transposed, for positions b0 .. b0 + 31:
    // each of the thread's 8 dimensions gets its 4 positions in one 8-byte store
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) k_lds[swz(4 * pgrp + pass, kpiece)] = kreg[pass];
    stage_v(vt_lds, vreg, kpiece, pgrp);
    if (b0 + kBlk < p_end) fetch(b0 + kBlk);            // uniform
    __syncthreads();

#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int mt = wave + 4 * i;
      if (mt >= MT) break;                             // uniform per wave
      attn_tile_block(p, q_lds, k_lds, vt_lds, b0, p_end, mt, col, quad, acc[i], m_run[i], l_run[i]);
    }
  }

  // The O^T tile holds (dim 16 d + 4 quad + j, row col) in lane (col, quad):
  // write the split's unnormalised rows, their maxima and sums.
  const int64_t base = ((int64_t)split * p.Hkv + kvh) * p.R;
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int mt = wave + 4 * i;
    if (mt >= MT) break;
    const int row = mt * 16 + col;
    if (row >= p.R) continue;
#pragma unroll
    for (int d = 0; d < 16; ++d)
      *reinterpret_cast<f32x4*>(p.ws_o + (base + row) * kD + 16 * d + 4 * quad) = acc[i][d];
    if (quad == 0) {
      p.ws_ml[(base + row) * 2] = m_run[i];
      p.ws_ml[(base + row) * 2 + 1] = l_run[i];
    }
  }
}

// Pass 2: one workgroup of 256 threads (one per dimension) per (KV head, row).
// Thread s < S takes split s's maximum and sum: the maximum over the splits
// and the normaliser sum_s 2^(m_s - M) l_s are workgroup reductions, and the
// weights 2^(m_s - M) go to LDS.  Each thread then adds its dimension of
// every split's row in split order, 16 loads in flight at a time.
constexpr int kMaxSplits = 256;   // attn_plan never makes more
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  const int kvh = blockIdx.y, row = blockIdx.x, dim = threadIdx.x, lane = dim & 63, wave = dim >> 6;
  __shared__ float wts[kMaxSplits];
  __shared__ float part[4];
  float ms = -__builtin_inff(), ls = 0.0f;
  if (dim < p.S) {
    const float2 v = *reinterpret_cast<const float2*>(p.ws_ml + (((int64_t)dim * p.Hkv + kvh) * p.R + row) * 2);
    ms = v.x;
    ls = v.y;
  }
  float M = wave_max(ms);
  if (lane == 0) part[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float w = ms > -__builtin_inff() ? __builtin_amdgcn_exp2f(ms - M) : 0.0f;
  if (dim < p.S) wts[dim] = w;
  float den = w * ls;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
  __syncthreads();                                   // part[] reads done, wts[] written
  if (lane == 0) part[wave] = den;
  __syncthreads();
  den = (part[0] + part[1]) + (part[2] + part[3]);
  float num = 0.0f;
  const float* src = p.ws_o + ((int64_t)kvh * p.R + row) * kD + dim;
  const int64_t sstride = (int64_t)p.Hkv * p.R * kD;        // between splits
#pragma unroll 16
  for (int s = 0; s < p.S; ++s) num += wts[s] * src[s * sstride];
  const int t = row / p.G, h = kvh * p.G + row % p.G;
  p.o[((int64_t)t * p.Hq + h) * kD + dim] = float_to_half_bits(num / den);
}

}  // namespace

AttnPlan attn_plan(int64_t T, int64_t Hq, int64_t Hkv, int64_t L) {
  AttnPlan pl;
  const int64_t G = Hq / Hkv, R = T * G;
  // About 256 workgroups in pass 1 (splits are a multiple of 32 positions,
  // at least one block).  Short caches get as many splits as they have
  // blocks: at 1.5k positions, 48 splits of one block ran in 14.6 us, 12
  // splits of four in 20.9 us (the per-split partial rows then outweigh the
  // cache, but pass 1 fills the GPU); with the current pass 1, 24 splits of
  // two took 13.5 us and 16 of three 12.5 us, against 12.6 us.  More than 256 workgroups made long
  // caches slower (16k positions: 44 us at 512 against 38 us), as pass 2
  // has more partial rows to read.
  int64_t S = std::max<int64_t>(1, std::min<int64_t>((256 + Hkv - 1) / Hkv, (L + kBlk - 1) / kBlk));
  int64_t C = ((L + S - 1) / S + kBlk - 1) / kBlk * kBlk;
  S = (L + C - 1) / C;
  pl.C = C;
  pl.S = S;
  pl.R = R;
  // row maxima and sums first (rounded up to 16 bytes), then the outputs
  pl.ml_floats = ((size_t)S * Hkv * R * 2 + 3) / 4 * 4;
  pl.ws_bytes = (pl.ml_floats + (size_t)S * Hkv * R * kD) * 4;
  return pl;
}

hipError_t launch_verify_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int64_t T,
                                   int64_t Hq, int64_t Hkv, int64_t L, void* ws, hipStream_t st) {
  const AttnPlan pl = attn_plan(T, Hq, Hkv, L);
  AttnParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.T = (int)T;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.G = (int)(Hq / Hkv);
  p.R = (int)pl.R;
  p.L = (int)L;
  p.C = (int)pl.C;
  p.S = (int)pl.S;
  p.ws_ml = reinterpret_cast<float*>(ws);
  p.ws_o = p.ws_ml + pl.ml_floats;
  const dim3 g1((unsigned)pl.S, (unsigned)Hkv);
  if ((pl.R + 15) / 16 > 4)
    attn_split_kernel<2><<<g1, dim3(256), 0, st>>>(p);
  else
    attn_split_kernel<1><<<g1, dim3(256), 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_combine_kernel<<<dim3((unsigned)pl.R, (unsigned)Hkv), dim3(256), 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace qg
