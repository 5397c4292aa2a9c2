// Weight-streaming GEMMs for small token counts (M <= 64): batched decode,
// speculative verify (M = 1 + draft tokens) and the int8 lm_head.
//
// Sources: "What this repo does that stock vLLM doesn't", "In full" items 4
// (W4A8: int8 activations x int4 weights, int32 accumulation per group,
// signed group scales) and 5 (the int8 lm_head read per draft); the project
// README, "What each step buys" (W4A16 body).  At these M the product reads
// each weight byte once and does little arithmetic per byte, so the kernel is
// built to keep HBM busy: every wavefront streams 1 KiB weight blocks with
// 128-bit buffer loads, several groups ahead of the matrix-core work.
//
// Work split.  A workgroup of NW wavefronts owns NT n-tiles (16 output
// columns = 16 rows of W each) over all of K; its waves take the K groups
// round-robin, so every weight and activation byte is read once per
// workgroup, and their fp32 sums meet in LDS and are added in wave order
// (results are bit-reproducible; no atomics), after which every thread
// stores part of the tile.  More waves per workgroup means fewer groups, and
// so fewer dependent memory round trips, per wave.
//
// Matrix-core mapping.  Weights are the A operand (rows n), activations the B
// operand (columns m), so a 16x16 output tile lands as 4 consecutive n for
// one m in each lane.  Per 128-wide group:
//   W4A8   2 x v_mfma_i32_16x16x64_i8 on (16*q_w, q_a) -> 16*P exactly, then
//          acc += fp32(16*P) * s_w; the token scale at the end carries the
//          1/16 (a power of two: the same result as scaling each term)
//   W4A16  4 x v_mfma_f32_16x16x32_f16 on the biased fp16 codes (1032 + q_w,
//          or 1152 + 16 q_w against x / 16) and fp16 x, started from minus
//          the activations' bias (4 more products with a constant operand,
//          shared by the stage's n-tiles), then acc += group_sum * s_w
//   W8A16  as W4A16 with int8 table codes converted exactly to fp16.
// The k order inside a lane operand is a permutation shared by both operands,
// so the contraction is unaffected by it.  W4A8 reads its activation codes
// in fragment order (see act_quant.hip): each 16-byte lane operand of a
// 16-row m-tile is contiguous, so one load instruction moves 1 KiB.
#include "common.h"
#include "operands.h"

namespace qg {
namespace {

struct SkinnyParams {
  const void* act;          // W4A8: codes in fragment order; else fp16 [M][lda]
  int64_t lda;
  const float* tok_scale;
  const void* w;
  const uint16_t* s;
  int M, N, K, G;
  int ms;                   // m-groups: workgroups that share an n-block, each with MT m-tiles
  int wgs;                  // n-blocks of unequal size (0: NT tiles each): block b has tiles
                            // [b T / wgs, (b + 1) T / wgs) of the T n-tiles, or, with t1,
  int t1;                   // the first wgs / 2 blocks share tiles [0, t1) and the rest [t1, T)
  uint16_t* y;
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

// One pipeline stage: one 128-wide group's weights and scales for the NT
// n-tiles of the workgroup and the matching activation fragments.
template <int MODE, int NT, int MT>
struct Stage;

template <int NT, int MT>
struct Stage<kW4A8, NT, MT> {
  uint4 w[NT];
  uint2 sc[NT];     // the lane's 4 fp16 group scales per n-tile
  i32x4 x[MT][2];
};

template <int NT, int MT>
struct Stage<kW4A16, NT, MT> {
  uint4 w[NT];
  f16x8 x[MT][4];
};

template <int NT, int MT>
struct Stage<kW8A16, NT, MT> {
  uint4 w[NT][2];
  f16x8 x[MT][4];
};

// Buffer resources over the bytes one workgroup may read.  Loads use the
// hardware range check: a row past M, an n-tile past N or a pipeline stage
// past the wave's last group is an out-of-range offset, which returns zeros
// without touching memory.  That keeps every load unconditional, so the
// prefetch ring is branch-free and the compiler counts outstanding loads
// exactly.
struct Rsrc {
  __amdgpu_buffer_rsrc_t w, s, x;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOOB = 0x80000000u;   // beyond every resource's extent (checked on the host)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Packed int4 weight loads: each 1 KiB block is read once per call, in full
// lines, so they carry the non-temporal hint (aux bit 1; measured 4-7%
// faster on the verify and int4 lm_head shapes and 2% on decode).  Not the
// int8 table rows: there the two 64-byte halves of a line arrive in two
// loads, and without the hint the line stays cached between them (with it,
// the draft head ran 44 -> 57 us).  Activations and scales keep the default
// policy: every workgroup reads them.
constexpr int kAuxStream = 2;
__device__ __forceinline__ uint4 ld128_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxStream));
}

template <int MODE, int NT, int MT, bool SL>
__device__ __forceinline__ void load_stage(const SkinnyParams& p, const Rsrc& rs, Stage<MODE, NT, MT>& st,
                                           bool valid, int g, int lane, int mt0) {
  const int col = lane & 15, quad = lane >> 4;
  const uint32_t G = (uint32_t)p.G;
  const uint32_t bad = valid ? 0u : kOOB;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if constexpr (MODE == kW8A16) {
      const uint32_t row = (uint32_t)(j * 16 + col) * (uint32_t)p.K + (uint32_t)g * kGroup + 16u * quad;
      st.w[j][0] = ld128(rs.w, row + bad);
      st.w[j][1] = ld128(rs.w, row + 64u + bad);
    } else {
      // packed block (n-tile j, group g) and the lane's 4 scales of it
      const uint32_t blk = (uint32_t)j * G + (uint32_t)g;
      st.w[j] = ld128_stream(rs.w, (blk * 64u + lane) * 16u + bad);
      if constexpr (MODE == kW4A8 && !SL)
        st.sc[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.s, (blk * 16u + 4u * quad) * 2u + bad, 0, 0));
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t m = (uint32_t)((mt0 + mt) * 16 + col);
    if constexpr (MODE == kW4A8) {
      const uint32_t off = ((((uint32_t)(mt0 + mt) * G + (uint32_t)g) * 2u) * 64u + lane) * 16u + bad;
      st.x[mt][0] = __builtin_bit_cast(i32x4, ld128(rs.x, off));
      st.x[mt][1] = __builtin_bit_cast(i32x4, ld128(rs.x, off + 1024u));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t off =
            (m * (uint32_t)p.lda + (uint32_t)g * kGroup + 64u * (t >> 1) + 16u * quad + 8u * (t & 1)) * 2u + bad;
        st.x[mt][t] = __builtin_bit_cast(f16x8, ld128(rs.x, off));
      }
    }
  }
}

// Group scales, fed to v_fma_mix as fp16.  W4A8 reads them from LDS in
// their memory layout, [n-tile][group][16 columns] (SL), or, when K is too
// long for that, from the stage, which then carries them.  W4A16 and W8A16
// read them from LDS, stored there as [group][column of the workgroup].  A
// stage past the wave's last group reads group 0's (its products are zero).
// W4A8 sums fp32(16 P) * s: the factor 16 of the 16*q weights is removed
// with the token scale at the end (an exact power of two, so the result is
// the same as scaling every term).
template <int MODE, int NT, int MT, bool DEBUG, bool SL>
__device__ __forceinline__ void compute_stage(const SkinnyParams& p, const Stage<MODE, NT, MT>& st, int g,
                                              bool gvalid, int nt0, int nvalid, int mt0, int lane,
                                              const uint16_t* lds_s, f32x4 (&acc)[NT][MT]) {
  const int col = lane & 15, quad = lane >> 4;
  const int gs = gvalid ? g : 0;
  // fp16 activation operands.  W4A16: the int4 conversion leaves every
  // weight value biased (see operands.h), so each m-tile's product starts
  // from minus the bias of its activation columns, formed once per stage by
  // the matrix core from the constant bias operand and shared by all
  // n-tiles.  W8A16 converts exactly and starts from zero.
  f16x8 b[MT][4];
  f32x4 seed[MT];
  if constexpr (MODE != kW4A8) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      seed[mt] = (f32x4)0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // W4A16 weight elements come in k order {0,2,4,6,1,3,5,7}; match it.
        if constexpr (MODE == kW4A16)
          b[mt][t] = w4_scale_activations(
              __builtin_shufflevector(st.x[mt][t], st.x[mt][t], 0, 2, 4, 6, 1, 3, 5, 7));
        else
          b[mt][t] = st.x[mt][t];
      }
      if constexpr (MODE == kW4A16) {
        const f16x8 c = w4_bias_operand();
#pragma unroll
        for (int t = 0; t < 4; ++t) seed[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(c, b[mt][t], seed[mt], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    uint2 sv;
    if constexpr (MODE == kW4A8 && !SL)
      sv = st.sc[j];
    else if constexpr (MODE == kW4A8)
      sv = *reinterpret_cast<const uint2*>(lds_s + (j * p.G + gs) * 16 + 4 * quad);
    else
      sv = *reinterpret_cast<const uint2*>(lds_s + gs * (16 * NT) + j * 16 + 4 * quad);
    const _Float16 sc[4] = {__builtin_bit_cast(_Float16, (uint16_t)(sv.x & 0xFFFFu)),
                            __builtin_bit_cast(_Float16, (uint16_t)(sv.x >> 16)),
                            __builtin_bit_cast(_Float16, (uint16_t)(sv.y & 0xFFFFu)),
                            __builtin_bit_cast(_Float16, (uint16_t)(sv.y >> 16))};
    if constexpr (MODE == kW4A8) {
      const i32x4 a0 = w4_to_i8x16(st.w[j].x, st.w[j].y);
      const i32x4 a1 = w4_to_i8x16(st.w[j].z, st.w[j].w);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        i32x4 P = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, st.x[mt][0], (i32x4)0, 0, 0, 0);
        P = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, st.x[mt][1], P, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][mt][r] = __builtin_fmaf((float)P[r], (float)sc[r], acc[j][mt][r]);
        if constexpr (DEBUG) {
          // tiles past nvalid belong to the next n-block (zero weights here)
          const int m = (mt0 + mt) * 16 + col;
          if (gvalid && j < nvalid && m >= p.dm0 && m < p.dm1 && m < p.M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int n = (nt0 + j) * 16 + 4 * quad + r;
              if (n >= p.dn0 && n < p.dn1 && n < p.N)
                p.dbg[((int64_t)(m - p.dm0) * (p.dn1 - p.dn0) + (n - p.dn0)) * p.G + g] = P[r] >> 4;
            }
          }
        }
      }
    } else {
      f16x8 a[4];
      if constexpr (MODE == kW4A16) {
        a[0] = w4_to_f16x8_biased(st.w[j].x);
        a[1] = w4_to_f16x8_biased(st.w[j].y);
        a[2] = w4_to_f16x8_biased(st.w[j].z);
        a[3] = w4_to_f16x8_biased(st.w[j].w);
      } else {
        a[0] = i8_to_f16x8(st.w[j][0].x, st.w[j][0].y);
        a[1] = i8_to_f16x8(st.w[j][0].z, st.w[j][0].w);
        a[2] = i8_to_f16x8(st.w[j][1].x, st.w[j][1].y);
        a[3] = i8_to_f16x8(st.w[j][1].z, st.w[j][1].w);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[mt][0], seed[mt], 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b[mt][1], gs, 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2], b[mt][2], gs, 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[3], b[mt][3], gs, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][mt][r] = __builtin_fmaf(gs[r], (float)sc[r], acc[j][mt][r]);
      }
    }
  }
}

// Epilogue of both weight-streaming kernels: the waves' fp32 sums meet in
// LDS (red, 2 x NW x QC x 64 f32x4 when the tiles take several chunks) and
// are added in wave order, then stored as fp16.  W4A8 (one m-tile, at most
// 40 KiB of sums) takes them in one chunk, so one barrier; the fp16 kernels
// keep their buffers within 32 KiB, which leaves LDS for their scales and a
// second workgroup per CU.
template <int MODE, int NT, int MT, int NW>
constexpr int red_chunk() {
  return MODE == kW4A8 || NT * MT * NW <= 32 ? NT * MT : 32 / NW;
}
template <int MODE, int NT, int MT, int NW>
constexpr int red_bufs() {
  return (NT * MT + red_chunk<MODE, NT, MT, NW>() - 1) / red_chunk<MODE, NT, MT, NW>() > 1 ? 2 : 1;
}

template <int MODE, int NT, int MT, int NW>
__device__ __forceinline__ void sum_and_store(const SkinnyParams& p, const f32x4 (&acc)[NT][MT], int nt0, int mt0,
                                              int nvalid, int wave, int lane,
                                              f32x4 (*red)[NW][red_chunk<MODE, NT, MT, NW>()][64]) {
  // Sum over the waves in wave order, QC (n-tile, m-tile) tiles at a time:
  // every wave parks its f32x4 per lane and tile in LDS, one barrier, then
  // thread t of a tile adds the 4 columns 4 (t % 4) .. + 3 of row t / 4 over
  // the waves and stores them, so consecutive threads write consecutive
  // bytes of a row.  Value (m, n) of a tile sits in lane m % 16 + 16 (n / 4),
  // stored at slot lane ^ (lane / 16 % 4) so that the four lanes of a row
  // fall in distinct LDS banks.  Two buffers alternate (one barrier per
  // chunk); nothing is stored to global memory before the last barrier.
  constexpr int Q = NT * MT;                                  // tiles per wave
  constexpr int QC = red_chunk<MODE, NT, MT, NW>();            // tiles per chunk
  constexpr int NCH = (Q + QC - 1) / QC;
  const int tid = (int)threadIdx.x;
  constexpr int KPC = (QC * 64 + 64 * NW - 1) / (64 * NW);     // sums per thread per chunk
  f32x4 out[NCH][KPC];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int b = NCH > 1 ? ch & 1 : 0;
#pragma unroll
    for (int qq = 0; qq < QC; ++qq) {
      const int q = ch * QC + qq, j = q / MT, mt = q % MT;
      if (q < Q) red[b][wave][qq][lane ^ ((lane >> 4) & 3)] = acc[j][mt];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KPC; ++k) {
      const int e = tid + 64 * NW * k;                        // (tile qq, row r, column quad c4)
      out[ch][k] = (f32x4)0.0f;
      if (e < QC * 64 && ch * QC + (e >> 6) < Q) {
        const int qq = e >> 6, r = (e & 63) >> 2, c4 = e & 3;
        const int l = r + 16 * c4;
        f32x4 v = red[b][0][qq][l ^ c4];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[b][w][qq][l ^ c4];
        out[ch][k] = v;
      }
    }
  }
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < KPC; ++k) {
      const int e = tid + 64 * NW * k;
      if (e >= QC * 64 || ch * QC + (e >> 6) >= Q) continue;
      const int q = ch * QC + (e >> 6), j = q / MT, mt = q % MT, r = (e & 63) >> 2, c4 = e & 3;
      const int m = (mt0 + mt) * 16 + r;
      if (m >= p.M || j >= nvalid) continue;
      // W4A8: token scale and the 1/16 of the 16*q weights
      const float ts = MODE == kW4A8 ? p.tok_scale[m] * 0.0625f : 1.0f;
      const f32x4 v = out[ch][k];
      uint2 o;
      o.x = (uint32_t)float_to_half_bits(v[0] * ts) | ((uint32_t)float_to_half_bits(v[1] * ts) << 16);
      o.y = (uint32_t)float_to_half_bits(v[2] * ts) | ((uint32_t)float_to_half_bits(v[3] * ts) << 16);
      *reinterpret_cast<uint2*>(p.y + (int64_t)m * p.N + (nt0 + j) * 16 + 4 * c4) = o;
    }
}

template <int MODE, int NT, int MT, int NW, int PF, bool DEBUG, bool SL>
__global__ __launch_bounds__(64 * NW) void skinny_kernel(SkinnyParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, in an SGPR
  // Workgroup -> (n-block, m-group).  With several m-groups the grid is
  // walked so that the m-groups of one n-block are consecutive on one XCD
  // (workgroups go to the XCDs round-robin): they run together, each on its
  // own 16 rows, and read the n-block's weights through that XCD's L2.
  int nb = blockIdx.x, mg = 0;
  if (p.ms > 1) {
    const unsigned total = gridDim.x, per = total >> 3;
    unsigned lin = blockIdx.x;
    if ((total & 7u) == 0 && per % (unsigned)p.ms == 0) lin = (blockIdx.x & 7u) * per + (blockIdx.x >> 3);
    nb = (int)(lin / (unsigned)p.ms);
    mg = (int)(lin % (unsigned)p.ms);
  }
  int nt0, nvalid;
  if (p.t1) {
    const int half = p.wgs / 2, T = p.N / 16;
    const int lo = nb < half ? 0 : p.t1, cnt = nb < half ? p.t1 : T - p.t1, b = nb < half ? nb : nb - half;
    nt0 = lo + (int)((int64_t)b * cnt / half);
    nvalid = lo + (int)((int64_t)(b + 1) * cnt / half) - nt0;
  } else {
    nt0 = p.wgs ? (int)((int64_t)nb * (p.N / 16) / p.wgs) : nb * NT;
    nvalid = p.wgs ? (int)((int64_t)(nb + 1) * (p.N / 16) / p.wgs) - nt0 : min(NT, p.N / 16 - nt0);
  }
  const int mt0 = mg * MT;

  f32x4 acc[NT][MT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x4)0.0f;

  Rsrc rs;
  {
    const int64_t G = p.G;
    if constexpr (MODE == kW8A16)
      rs.w = make_rsrc(reinterpret_cast<const int8_t*>(p.w) + (int64_t)nt0 * 16 * p.K,
                       (uint32_t)(nvalid * 16 * (int64_t)p.K));
    else
      rs.w = make_rsrc(reinterpret_cast<const uint8_t*>(p.w) + (int64_t)nt0 * G * 1024, (uint32_t)(nvalid * G * 1024));
    if constexpr (MODE == kW4A8)
      rs.x = make_rsrc(p.act, (uint32_t)((int64_t)((p.M + 15) / 16) * 16 * p.K));
    else
      rs.x = make_rsrc(p.act, (uint32_t)(((int64_t)(p.M - 1) * p.lda + p.K) * 2));
    rs.s = make_rsrc(p.s + (int64_t)nt0 * G * 16, (uint32_t)(nvalid * G * 32));
  }

  // The workgroup's group scales (NT*16 columns x G groups, one contiguous
  // block in both scale layouts) go to LDS once.  W4A16 / W8A16: through
  // registers, transposed to [group][column]; the loads are issued before
  // the weight prefetch so the barrier below waits for them only.  W4A8
  // (SL): as they lie in memory, by LDS-direct loads of 1 KiB per wave
  // issued before the first stage, so they travel with it; this takes the
  // small scale loads (one per n-tile and group) off the load path that
  // bounds the decode kernel.
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_s[];
  constexpr int COLS = 16 * NT;
  constexpr int SPT = 8;                       // scales per thread per pass (one 16-byte load)
  uint4 sreg[4];
  int nsc = 0, npass = 0;
  const uint16_t* sbase = p.s + (int64_t)nt0 * 16 * p.G;   // same block start in both layouts
  // scale index -> (column, group) in the block
  auto scol = [&](int idx) { return MODE == kW8A16 ? idx / p.G : (idx / (16 * p.G)) * 16 + idx % 16; };
  auto sgrp = [&](int idx) { return MODE == kW8A16 ? idx % p.G : (idx / 16) % p.G; };
  if constexpr (MODE != kW4A8) {
    nsc = nvalid * 16 * p.G;                   // scales of the valid columns
    npass = (nsc + 64 * NW * SPT - 1) / (64 * NW * SPT);
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(sbase, (uint32_t)nsc * 2u);
#pragma unroll
    for (int i = 0; i < 4; ++i) sreg[i] = ld128(srs, (uint32_t)(threadIdx.x + 64 * NW * i) * SPT * 2u);
    for (int i = 4; i < npass; ++i) {          // very long K: load and store directly
      const int e = (threadIdx.x + 64 * NW * i) * SPT;
      if (e < nsc) {
        const uint4 v = *reinterpret_cast<const uint4*>(sbase + e);
        const uint16_t h[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                               (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int idx = e + t;
          lds_s[sgrp(idx) * COLS + scol(idx)] = h[t];
        }
      }
    }
  }
  if constexpr (MODE == kW4A8 && SL) {
    const int nchunk = (nvalid * p.G * 32 + 1023) >> 10;   // the dynamic LDS holds ceil(NT G 32 / 1024) KiB
    for (int c = wave; c < nchunk; c += NW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.s, (lds_ptr_t)(lds_s + c * 512), 16, (uint32_t)lane * 16u,
                                               (uint32_t)c * 1024u, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // This wave's groups are wave, wave + NW, ...; PF of them are in flight in
  // a register ring.  Scheduling barriers keep each stage's multiply after
  // the previous stage's loads, so a stage waits only for its own data.  The
  // last round issues no loads, so nothing is fetched past the last group.
  const int ng = wave < p.G ? (p.G - wave + NW - 1) / NW : 0;
  const int rounds = (ng + PF - 1) / PF;
  // Each n-block walks its wave's groups from a different starting point,
  // so concurrent workgroups do not all read the same activation columns
  // (the same L2 lines) at the same moment.  The m-groups of an n-block
  // share the starting point: they then ask for the same weight lines
  // together (staggering them was measured slower), and a row's sum order
  // does not depend on how M is split.
  const int rot = ng > 0 ? nb % ng : 0;
  auto gidx = [&](int i) { return wave + NW * (i < ng ? (i + rot < ng ? i + rot : i + rot - ng) : i); };
  Stage<MODE, NT, MT> st[PF];
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    load_stage<MODE, NT, MT, SL>(p, rs, st[s], s < ng, gidx(s), lane, mt0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (MODE == kW4A8 && SL) {
    // Loads complete in order: once no more than the ring's own loads are
    // outstanding, this wave's scale chunks are in LDS.  A bare barrier
    // between compiler fences then publishes them; a release fence would
    // also wait for the ring.
    constexpr int kRing = PF * (NT + 2 * MT);
    static_assert(kRing < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((kRing & 15) | ((kRing >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  if constexpr (MODE != kW4A8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = (threadIdx.x + 64 * NW * i) * SPT;
      if (i < npass && e < nsc) {
        const uint16_t h[8] = {(uint16_t)sreg[i].x, (uint16_t)(sreg[i].x >> 16), (uint16_t)sreg[i].y,
                               (uint16_t)(sreg[i].y >> 16), (uint16_t)sreg[i].z, (uint16_t)(sreg[i].z >> 16),
                               (uint16_t)sreg[i].w, (uint16_t)(sreg[i].w >> 16)};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int idx = e + t;
          lds_s[sgrp(idx) * COLS + scol(idx)] = h[t];
        }
      }
    }
    __syncthreads();
  }

  for (int r = 0; r + 1 < rounds; ++r) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int ii = r * PF + s;
      compute_stage<MODE, NT, MT, DEBUG, SL>(p, st[s], gidx(ii), true, nt0, nvalid, mt0, lane, lds_s, acc);
      // Stages past the last group load nothing (out-of-range offsets) and
      // multiply zeros, which keeps this loop free of branches.
      load_stage<MODE, NT, MT, SL>(p, rs, st[s], ii + PF < ng, gidx(ii + PF), lane, mt0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (rounds > 0) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int ii = (rounds - 1) * PF + s;
      compute_stage<MODE, NT, MT, DEBUG, SL>(p, st[s], gidx(ii), ii < ng, nt0, nvalid, mt0, lane, lds_s, acc);
    }
  }

  __shared__ f32x4 red[red_bufs<MODE, NT, MT, NW>()][NW][red_chunk<MODE, NT, MT, NW>()][64];
  sum_and_store<MODE, NT, MT, NW>(p, acc, nt0, mt0, nvalid, wave, lane, red);
}

// W4A8 at 16 < M <= 64: the streaming kernel with the rows split over
// workgroups (see launch_skinny): n-blocks of 2 or 3 n-tiles, one or two
// 16-row m-tiles per workgroup, 8 waves, a one-stage ring.
constexpr int kMsplitNT = 3, kMsplitNW = 8, kMsplitPF = 1;
constexpr int kMsplitMinBlocks = 128;   // with two m-groups each, one workgroup per CU
constexpr int kBalancedWgs = 512;   // two workgroups per CU

// Prefetch depth: deep enough to keep several 1 KiB weight blocks per wave
// in flight, shallow enough to leave room for two waves per SIMD.
template <int MODE, int NT, int MT>
constexpr int prefetch_depth() {
  return MODE == kW4A8 ? (NT * MT <= 4 ? 5 : 3) : 2;
}

// W4A8 group scales staged in LDS: the bytes the kernel's LDS-direct loads
// fill (whole KiB), or 0 when K is too long for the budget, in which case
// the stages carry the scales.
constexpr size_t kScaleLdsMax = 32768;
inline size_t w4a8_scale_lds(int nt, int G) {
  const size_t b = ((size_t)32 * nt * G + 1023) / 1024 * 1024;
  return b <= kScaleLdsMax ? b : 0;
}

template <int MODE, int NT, int NW, bool DEBUG>
void launch_mt(const SkinnyParams& p, int mt, dim3 grid, hipStream_t st) {
  const dim3 block(64 * NW);
  if constexpr (MODE == kW4A8) {
    // M <= 16 here (larger W4A8 batches take the row split): one m-tile
    (void)mt;
    constexpr int PF = prefetch_depth<MODE, NT, 1>();
    if (const size_t lds = w4a8_scale_lds(NT, p.G))
      skinny_kernel<MODE, NT, 1, NW, PF, DEBUG, true><<<grid, block, lds, st>>>(p);
    else
      skinny_kernel<MODE, NT, 1, NW, PF, DEBUG, false><<<grid, block, 0, st>>>(p);
  } else {
    // the workgroup's group scales (K <= 65536 keeps this within 64 KiB)
    const size_t lds = (size_t)16 * NT * p.G * 2;
    switch (mt) {
      case 1: skinny_kernel<MODE, NT, 1, NW, prefetch_depth<MODE, NT, 1>(), DEBUG, false><<<grid, block, lds, st>>>(p); break;
      case 2: skinny_kernel<MODE, NT, 2, NW, prefetch_depth<MODE, NT, 2>(), DEBUG, false><<<grid, block, lds, st>>>(p); break;
      case 3: skinny_kernel<MODE, NT, 3, NW, prefetch_depth<MODE, NT, 3>(), DEBUG, false><<<grid, block, lds, st>>>(p); break;
      default: skinny_kernel<MODE, NT, 4, NW, prefetch_depth<MODE, NT, 4>(), DEBUG, false><<<grid, block, lds, st>>>(p); break;
    }
  }
}

template <int MT>
void launch_rowsplit(const SkinnyParams& p, bool dbg, size_t lds, dim3 grid, hipStream_t st) {
  constexpr int NT = kMsplitNT, NW = kMsplitNW, PF = kMsplitPF;
  if (dbg && lds)
    skinny_kernel<kW4A8, NT, MT, NW, PF, true, true><<<grid, dim3(64 * NW), lds, st>>>(p);
  else if (dbg)
    skinny_kernel<kW4A8, NT, MT, NW, PF, true, false><<<grid, dim3(64 * NW), 0, st>>>(p);
  else if (lds)
    skinny_kernel<kW4A8, NT, MT, NW, PF, false, true><<<grid, dim3(64 * NW), lds, st>>>(p);
  else
    skinny_kernel<kW4A8, NT, MT, NW, PF, false, false><<<grid, dim3(64 * NW), 0, st>>>(p);
}

// Two n-tiles per workgroup only for W4A8 (skinny_plan); every mode takes
// four on wide outputs.
template <int MODE, bool DEBUG>
hipError_t launch_mode(const SkinnyParams& p, const SkinnyPlan& pl, int mt, dim3 grid, hipStream_t st) {
  if constexpr (MODE == kW4A8) {
    if (pl.nt == 2) {
      launch_mt<MODE, 2, 4, DEBUG>(p, mt, grid, st);
      return hipGetLastError();
    }
  }
  launch_mt<MODE, 4, 4, DEBUG>(p, mt, grid, st);
  return hipGetLastError();
}

}  // namespace

SkinnyPlan skinny_plan(int mode, int64_t N, int64_t K) {
  (void)K;
  const int64_t ntiles = N / 16;
  SkinnyPlan pl;
  // Few output tiles (W4A8 at M <= 16 on decode-sized N): two n-tiles per
  // workgroup, so enough workgroups exist, and four waves splitting K, each
  // with a 5-deep ring (at M = 16, N = 5120: 5.5 us against 5.9 us with
  // eight waves, 5.7 us with two, 5.8 us with a ring of 3 or 4; one n-tile
  // with eight waves 6.7 us).  Many tiles (wide projections, the lm_head):
  // four n-tiles per workgroup, four waves.
  if (mode == kW4A8 && ntiles <= 1024)
    pl.nt = 2;
  else
    pl.nt = 4;
  return pl;
}

hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.dbg == nullptr && wide_waves(a.mode, a.M, a.N) != 0) return launch_wide(a, st);
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
  p.y = a.y;
  p.dbg = a.dbg;
  p.dm0 = (int)a.dm0; p.dm1 = (int)a.dm1; p.dn0 = (int)a.dn0; p.dn1 = (int)a.dn1;
  p.ms = 1;
  p.wgs = 0;
  p.t1 = 0;
  // W4A8 at 16 < M <= 64 (decode batches): the n-tiles dealt into
  // ceil(2T / 5) balanced n-blocks of 2 or 3 (at least min(T, 128) blocks,
  // so that narrow outputs still fill the CUs: at N = 1024, 2048 and 3072
  // that took M = 64 from 8.1, 8.3 and 8.5 us to 6.4, 6.5 and 7.1 us), and
  // each n-block's rows split into m-groups of one 16-row m-tile (M <= 32)
  // or two (M > 32), so that M = 17 .. 64 all make two m-groups per n-block
  // at most (and the same n-blocks); 8 waves split K
  // with a one-stage ring.  Each CU then pulls 164 KB of activation codes
  // and 82-123 KB of weights at M = 64, K = N = 5120 (mostly L2 hits: the
  // n-block's two m-groups run on one XCD and share its weights), where one
  // m-tile over blocks of 4 or 5 n-tiles pulled 82 KB of codes and 200 KB
  // of weights shared four ways; the CU's limit on outstanding L2 requests
  // is what bounds this GEMM.  Measured at K = N = 5120: 7.9 us at M = 64
  // (8.1 us for the layout of 5 n-tiles x 16 rows), 7.4 us at M = 48
  // (8.1), 6.6 us at M = 17 .. 32 (8.2: that layout left half the CUs
  // idle), against 10.3 us for an LDS-slab kernel of two n-tiles x 64 rows
  // with every load in flight at once and 10.9 us for the streaming
  // kernel's two n-tiles x 64 rows.  One m-tile per workgroup on these
  // n-blocks (512 workgroups at M = 64) took 9.4 us; 4, 10 or 16 waves
  // 8.0-8.1 us; a deeper or earlier-issued ring is slower.  Every m-group
  // of an n-block walks the same groups in the same order, so a row's sum
  // does not depend on M here.  The debug window runs the same kernel,
  // instantiated with the partial-sum stores.
  if (a.mode == kW4A8 && a.M > 16) {
    const int mtpw = a.M > 32 ? 2 : 1;
    p.ms = (p.M + 16 * mtpw - 1) / (16 * mtpw);
    p.wgs = std::max((2 * (p.N / 16) + 4) / 5, std::min(p.N / 16, kMsplitMinBlocks));
    const dim3 grid((unsigned)(p.wgs * p.ms));
    const size_t lds = w4a8_scale_lds(kMsplitNT, p.G);
    if (mtpw == 2)
      launch_rowsplit<2>(p, a.dbg != nullptr, lds, grid, st);
    else
      launch_rowsplit<1>(p, a.dbg != nullptr, lds, grid, st);
    return hipGetLastError();
  }
  const SkinnyPlan pl = skinny_plan(a.mode, a.N, a.K);
  const int mt = (p.M + 15) / 16;
  // fp16-activation products over 1024 .. 2560 n-tiles (the verify
  // projections, the draft head): blocks of four n-tiles leave some CUs
  // with one workgroup more than the rest (544 workgroups for N = 34,816),
  // and those set the time; 512 blocks of four or five tiles give every CU
  // two.  The two are blocks b and b + 256, and the older one's waves issue
  // first: with equal blocks, per-workgroup timestamps at N = 34,816, M = 8
  // put the first 256 blocks' ends at a median of 13.6 us and the others'
  // at 16.6 us, the CU then running one workgroup alone.  The first 256
  // blocks therefore take 10/17 of the tiles, at most 5 each (5 against 3.5
  // tiles at that N; verify 18.8 -> 18.1 us at M = 8, 22.2 -> 21.2 us at
  // M = 16; 6 against 2.5 and 7 against 1.5 were slower).  Any split is a
  // partition of the tiles, so results do not depend on where the
  // workgroups land.
  if (a.mode != kW4A8 && a.dbg == nullptr && pl.nt == 4 && p.N / 16 > 1024 && p.N / 16 <= 5 * kBalancedWgs) {
    p.wgs = kBalancedWgs;
    p.t1 = std::min((int)((int64_t)(p.N / 16) * 10 / 17), 5 * (kBalancedWgs / 2));
    if (a.mode == kW4A16)
      launch_mt<kW4A16, 5, 4, false>(p, mt, dim3((unsigned)kBalancedWgs), st);
    else
      launch_mt<kW8A16, 5, 4, false>(p, mt, dim3((unsigned)kBalancedWgs), st);
    return hipGetLastError();
  }
  // Narrow outputs: blocks of pl.nt n-tiles would leave most CUs idle.
  // W4A16 / W8A16: where they would make fewer than 256 workgroups, the
  // n-tiles are dealt into 256 balanced blocks instead (one n-tile or more
  // each).  At M = 8 / 16: N = 1024 8.6 / 10.0 -> 8.0 / 8.8 us, N = 5120
  // 8.9 / 10.4 -> 8.5 / 9.4 us (512 blocks: 11.5 / 14.2 us at N = 5120).
  // W4A8 at M <= 16 gains only from equal blocks: one n-tile per workgroup
  // up to 256 n-tiles (M = 16: N = 1024 5.0 -> 4.5 us, N = 3072 5.3 ->
  // 4.8 us), while 128 blocks of one or two tiles took 5.5 us at N = 3072
  // and 256 of them 5.6 us at N = 5120, where its 160 two-tile blocks stay
  // (5.5 us).  The blocks depend on N only, so a row's sums do not depend
  // on M.
  dim3 grid((unsigned)((p.N / 16 + pl.nt - 1) / pl.nt));
  if ((int)grid.x < 256 && (a.mode != kW4A8 || p.N / 16 <= 256)) {
    p.wgs = std::min(p.N / 16, 256);
    grid = dim3((unsigned)p.wgs);
  }
  switch (a.mode) {
    case kW4A8:
      return a.dbg ? launch_mode<kW4A8, true>(p, pl, mt, grid, st) : launch_mode<kW4A8, false>(p, pl, mt, grid, st);
    case kW4A16: return launch_mode<kW4A16, false>(p, pl, mt, grid, st);
    default: return launch_mode<kW8A16, false>(p, pl, mt, grid, st);
  }
}

}  // namespace qg
