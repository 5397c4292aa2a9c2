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
// tiles of 16 x 16.  Per 128-wide group the workgroup stages in LDS the int8
// activation codes (128 rows x 128 B), the packed int4 weights (8 n-tiles x
// 1 KiB, already in lane order) and the 128 group scales, double buffered,
// with LDS-direct buffer loads: the data goes from memory straight into LDS
// (16 B per lane at consecutive addresses), so staging takes no registers
// and no LDS store instructions.  The next group's loads are issued before
// the current group's matrix-core work; one barrier per group.
//
// Activation layout in LDS.  Row r holds its 8 16-byte parts at slots
// part ^ ((r / 2) % 8), so the 16 rows a 16x16 tile's lanes read at one
// part fall in 16 distinct groups of 4 banks.
//
// Rescale.  Per group and tile two v_mfma_i32_16x16x64_i8 give 16 * P
// exactly, started from the bits of C = 1.5 * 2^23 so that the int32 result
// read as fp32 is C + 16 P; then acc += (C + 16 P) * s (fp16 scale operand
// of v_fma_mix) with no int-to-float conversion, and the bias C * s is
// taken off every four groups (below).  The factor 1/16 joins the token
// scale in the epilogue.  That is one vector FMA per output element and
// group plus a quarter for the bias; one wave sums the window's scales for
// the whole workgroup and shares them through LDS.  Within a group the
// tiles are software-pipelined (each tile's products go out around the
// previous tile's rescale).  The kernel is sized for three workgroups per
// CU (at most 168 VGPRs, 49 KiB of LDS).  Under this load the part runs
// at its power limit (about 2.0-2.2 GHz), so every instruction and byte
// moved per group costs time.
//
// Placement.  Workgroups are dealt to the 8 XCDs round-robin; ids are
// remapped so each XCD walks a contiguous run of a grouped tile order (8
// m-blocks by the n-blocks), and the workgroups resident together on an XCD
// share activation and weight slices in its L2.
#include <type_traits>

#include "common.h"

namespace qg {
namespace {

constexpr int BM = 128, BN = 128, GROUP_M = 8;
constexpr uint32_t kHiNib = 0xF0F0F0F0u;

// Conversion-free rescale.  Each group's first MFMA starts from the int32
// bits of C = 1.5 * 2^23 instead of zero, so the group's result, read as
// fp32, is exactly C + 16 P (|16 P| <= 16 * 127 * 8 * 128 < 2^22 keeps it
// in C's binade, where consecutive integers are consecutive floats).  Then
// acc += (C + 16 P) * s needs no int-to-float conversion; the bias C * s is
// summed per column and taken off every kBiasGroups groups, before it grows
// large enough to cost the accumulator precision.  On the prefill workload
// the fp16 outputs' relative Frobenius error against the float64 reference
// is 2.5e-4 (2.1e-4 with a conversion per group; 2.9e-4 with the bias taken
// off every 8 groups; the bound is 5e-4).
constexpr int32_t kBiasBits = 0x4B400000;
constexpr float kBias = 12582912.0f;
constexpr int kBiasGroups = 4;

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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// lo += fp32(low half of h), hi += fp32(high half of h), h two fp16: one
// mixed-precision FMA each (x * 1.0 + acc with x read as fp16), where the
// compiler would otherwise convert and add in two instructions.
__device__ __forceinline__ void add_f16_pair(float& lo, float& hi, uint32_t h) {
  asm("v_fma_mix_f32 %0, %2, 1.0, %0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %1, %2, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(lo), "+v"(hi)
      : "v"(h));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS-direct load: lane l's `size` bytes from rsrc + voff + soff land at
// lds + size * l.  Out-of-range offsets store zeros.
__device__ __forceinline__ void ld_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void ld_lds4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}

template <bool DEBUG>
__global__ __launch_bounds__(256, 3) void w4a8_large_kernel(LargeParams p) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint4 Bs[2][8 * 64];
  __shared__ __attribute__((aligned(16))) uint32_t Ss[2][64];   // 128 fp16 scales: [n-tile][16]
  // Per column: the scale sum of a bias window (below), alternating between
  // two buffers so that a window ending one group after another cannot
  // overwrite sums that other waves are still reading.
  __shared__ __attribute__((aligned(16))) float WS[2][128];

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

  // Range-checked resources: rows past M and n-tiles past N read zeros.
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.codes + (int64_t)m0 * p.K, (uint32_t)(mrows * (int64_t)p.K));
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(p.w + (int64_t)nt_base * G * 1024, (uint32_t)(nvt * (int64_t)G * 1024));
  const __amdgpu_buffer_rsrc_t rsS = make_rsrc(p.s + (int64_t)nt_base * G * 16, (uint32_t)(nvt * (int64_t)G * 32));

  // Per-lane offsets of the staging loads (the group adds a scalar offset).
  // A: wave w loads 1 KiB chunks c = 4w .. 4w+3 (rows 8c .. 8c+7); lane l
  // fills row 8c + l/8, slot l%8 with part (l%8) ^ ((row/2) % 8).
  // Chunks i and i + 2 are 16 rows apart, which leaves the swizzle
  // unchanged: they share a lane offset and differ by a scalar 16 K.
  uint32_t va[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (4 * wave + i) + (lane >> 3);
    va[i] = (uint32_t)r * (uint32_t)p.K + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  const uint32_t a_step = 16u * (uint32_t)p.K;
  // B: wave w loads n-tiles 2w, 2w+1 (one 1 KiB block each, G KiB apart).
  const uint32_t vb = ((uint32_t)(2 * wave) * (uint32_t)G * 64u + lane) * 16u;
  const uint32_t b_step = (uint32_t)G * 1024u;
  // S (wave 0): lane l loads scales 2(l%8), +1 of n-tile l/8.
  const uint32_t vs = (((uint32_t)(lane >> 3) * (uint32_t)G) * 16u + 2u * (lane & 7)) * 2u;

  auto gload = [&](int g, int8_t* A, uint4* B, uint32_t* S) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ld_lds16(rsA, A + (4 * wave + i) * 1024, va[i & 1], (uint32_t)g * 128u + (uint32_t)(i >> 1) * a_step);
#pragma unroll
    for (int i = 0; i < 2; ++i) ld_lds16(rsB, B + (2 * wave + i) * 64, vb, (uint32_t)g * 1024u + (uint32_t)i * b_step);
    if (wave == 0) ld_lds4(rsS, S, vs, (uint32_t)g * 32u);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[j][mt] = (f32x4)0.0f;
  // Wave 0 sums each window's scales for the whole workgroup, two columns
  // per lane (word `lane` of a scale stage: columns 2 lane, 2 lane + 1).
  float ws0 = 0.0f, ws1 = 0.0f;

  // LDS byte offsets of this lane's activation operands: m-tile mt, half h
  // (k 64h + 16 quad .. +15 of the group = part 4h + quad).
  uint32_t xoff[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int rr = wm * 64 + mt * 16 + col;
#pragma unroll
    for (int h = 0; h < 2; ++h) xoff[mt][h] = (uint32_t)rr * 128u + 16u * (uint32_t)((4 * h + quad) ^ ((rr >> 1) & 7));
  }

  gload(0, As[0], Bs[0], Ss[0]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // One group g whose operands sit in stage BUF (a constant: the loop runs
  // two groups per iteration, so the LDS addresses of both stages are fixed
  // offsets and cost no vector instructions).
  auto group = [&](int g, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    // All of this group's operands come out of LDS first; only then are the
    // next group's LDS-direct loads issued (into the other stage), so no
    // LDS read of this group waits behind them.
    i32x4 xb[4][2];
    uint4 wv[4];
    uint2 sv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) xb[mt][h] = *reinterpret_cast<const i32x4*>(&As[buf][xoff[mt][h]]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wv[j] = Bs[buf][(wn * 4 + j) * 64 + lane];
      sv[j] = *reinterpret_cast<const uint2*>(&Ss[buf][(wn * 4 + j) * 8 + 2 * quad]);
    }
    const bool window_end = (g % kBiasGroups) == kBiasGroups - 1 || g == G - 1;
    float* const wsum_buf = WS[(g / kBiasGroups) & 1];
    if (wave == 0) {
      add_f16_pair(ws0, ws1, Ss[buf][lane]);
      if (window_end) {
        *reinterpret_cast<float2*>(&wsum_buf[2 * lane]) = float2{ws0, ws1};
        ws0 = 0.0f;
        ws1 = 0.0f;
      }
    }
    if (g + 1 < G) gload(g + 1, As[buf ^ 1], Bs[buf ^ 1], Ss[buf ^ 1]);

    // Software pipeline over the 16 tiles t = (n-tile j, m-tile mt): tile
    // t's two matrix-core products go out around tile t - 1's rescale and a
    // quarter of the next n-tile's unpack, so that vector work issues while
    // the matrix core runs instead of waiting for the product it reads.
    // Scheduling barriers hold that order; the empty asm on each rescaled
    // accumulator keeps the compiler from sinking the rescales to the end
    // of the group (where all 16 products would be live at once).
    auto unpack_half = [&](uint32_t w, i32x4& a, int k) {
      a[2 * k] = (int32_t)((w << 4) & kHiNib);
      a[2 * k + 1] = (int32_t)(w & kHiNib);
    };
    auto scale = [&](int j, int r) -> float {
      const uint32_t h = (r < 2) ? sv[j].x : sv[j].y;
      return (float)__builtin_bit_cast(_Float16, (uint16_t)((r & 1) ? (h >> 16) : (h & 0xFFFFu)));
    };
    i32x4 wa[2][2];   // unpacked int8 operands (16 q) of n-tiles j and j + 1
    unpack_half(wv[0].x, wa[0][0], 0);
    unpack_half(wv[0].y, wa[0][0], 1);
    unpack_half(wv[0].z, wa[0][1], 0);
    unpack_half(wv[0].w, wa[0][1], 1);
    i32x4 Pp;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int j = t >> 2, mt = t & 3;
      const int jp = (t - 1) >> 2, mp = (t - 1) & 3;
      __builtin_amdgcn_sched_barrier(0);
      i32x4 P = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[j & 1][0], xb[mt][0], (i32x4)kBiasBits, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (t > 0) {
        // The whole vector is reinterpreted at once: taking element r of the
        // int vector and then its bits as float made the compiler feed
        // element 0 to all four mixed-precision FMAs.
        const f32x4 F = __builtin_bit_cast(f32x4, Pp);
        acc[jp][mp][0] = __builtin_fmaf(F[0], scale(jp, 0), acc[jp][mp][0]);
        acc[jp][mp][1] = __builtin_fmaf(F[1], scale(jp, 1), acc[jp][mp][1]);
        asm volatile("" : "+v"(acc[jp][mp]));
      }
      __builtin_amdgcn_sched_barrier(0);
      P = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[j & 1][1], xb[mt][1], P, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (t > 0) {
        const f32x4 F = __builtin_bit_cast(f32x4, Pp);
        acc[jp][mp][2] = __builtin_fmaf(F[2], scale(jp, 2), acc[jp][mp][2]);
        acc[jp][mp][3] = __builtin_fmaf(F[3], scale(jp, 3), acc[jp][mp][3]);
        asm volatile("" : "+v"(acc[jp][mp]));
      }
      if (j < 3) {
        const uint32_t w = mt == 0 ? wv[j + 1].x : mt == 1 ? wv[j + 1].y : mt == 2 ? wv[j + 1].z : wv[j + 1].w;
        unpack_half(w, wa[(j + 1) & 1][mt >> 1], mt & 1);
      }
      if constexpr (DEBUG) {
        const int m = m0 + wm * 64 + mt * 16 + col;
        if (m >= p.dm0 && m < p.dm1 && m < p.M) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = (nt_base + wn * 4 + j) * 16 + 4 * quad + r;
            if (n >= p.dn0 && n < p.dn1 && n < p.N)
              p.dbg[((int64_t)(m - p.dm0) * (p.dn1 - p.dn0) + (n - p.dn0)) * G + g] = (P[r] - kBiasBits) >> 4;
          }
        }
      }
      Pp = P;
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      const f32x4 F = __builtin_bit_cast(f32x4, Pp);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[3][3][r] = __builtin_fmaf(F[r], scale(3, r), acc[3][3][r]);
    }
    // This wave's loads for group g + 1 have landed; after the barrier,
    // every wave's have, nobody reads this stage any more, and a window that
    // ended here has its sums in LDS.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Take off the window's bias: C times each column's scale sum.
    if (window_end) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 wsum = *reinterpret_cast<const f32x4*>(&wsum_buf[(wn * 4 + j) * 16 + 4 * quad]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][mt][r] = __builtin_fmaf(-kBias, wsum[r], acc[j][mt][r]);
      }
    }
  };
  int g = 0;
  for (; g + 2 <= G; g += 2) {
    group(g, std::integral_constant<int, 0>{});
    group(g + 1, std::integral_constant<int, 1>{});
  }
  if (g < G) group(g, std::integral_constant<int, 0>{});

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
