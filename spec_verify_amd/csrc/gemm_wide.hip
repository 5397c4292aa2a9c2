// Weight-streaming GEMM for wide outputs with fp16 activations (M <= 64):
// the verify-sized W4A16 projections and the int8 lm_head over the
// vocabulary table (W8A16).
//
// Sources: "What this repo does that stock vLLM doesn't", "In full" items 1
// and 5 (the int8 lm_head read per draft); the project README, "What each
// step buys" (the W4A16 body).  The product reads each weight byte once;
// what else a CU reads decides how close it gets to the HBM rate.
//
// Work split.  A workgroup of NW wavefronts owns NW * TPW n-tiles (16 output
// columns each); each wave streams its own TPW n-tiles over all of K and
// keeps their sums, so no partial sums ever cross waves.  The fp16
// activations of each 128-wide group are staged once per workgroup in LDS,
// so the M x K activations pass through a CU once per NW * TPW n-tiles; with
// K split across waves instead (the weight-streaming kernel for narrower
// outputs) every 4 n-tiles re-read them, and at M = 64 that is twice the
// weight bytes.
//
// Pipeline.  A ring of PF stages per wave: the weights of a group go to
// registers (range-checked buffer loads), its activations and the wave's
// own scales to an LDS slot (LDS-direct loads: memory to LDS, 16 B per lane
// at consecutive addresses).  Each wave issues the same loads per stage in a
// fixed order, so one counted s_waitcnt per group waits for exactly that
// group and leaves the next PF - 1 stages in flight; then one barrier per
// group.  (Waiting for a later load would drain every earlier one: loads
// complete in order.)
//
// Per group and tile: fp16 operands from the exact int4 / int8 codes
// (operands.h), 4 x v_mfma_f32_16x16x32_f16 into a group sum, then
// acc += group_sum * scale; groups are added in order 0, 1, ... per output.
#include "common.h"
#include "operands.h"

namespace qg {
namespace {

constexpr uint32_t kOOB = 0x80000000u;      // beyond every resource's extent (checked on the host)

struct WideParams {
  const uint16_t* x;      // fp16 [M][lda]
  int64_t lda;
  const void* w;          // packed int4 (W4A16) or row-major int8 [N][K] (W8A16)
  const uint16_t* s;      // packed scales [tile][G][16] (W4A16) or row-major fp16 [N][G] (W8A16)
  int M, N, K, G;
  uint16_t* y;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Packed int4 weights are read once per call, in full lines: non-temporal
// hint (aux bit 1).  The int8 table rows keep the default policy (the two
// halves of a line arrive in two loads).
__device__ __forceinline__ uint4 ld128_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// LDS-direct loads: lane l's bytes from r + voff + soff land at lds + 16 l
// (16-byte loads) or lds + 4 l (4- and 2-byte loads; a 2-byte value is
// zero-extended into its 4-byte slot); out-of-range offsets store zeros.
__device__ __forceinline__ void lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds2(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 2, voff, soff, 0, 0);
}

// s_waitcnt with vmcnt <= n and the other counters left alone (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
// s_waitcnt with vmcnt <= n and lgkmcnt = 0 (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4 left alone, lgkmcnt 11:8).
#define QG_WAIT_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))
// Keeps the compiler from moving memory accesses across this point; emits nothing.
#define QG_COMPILER_FENCE() asm volatile("" ::: "memory")

template <int MODE, int TPW>
struct WStage;
template <int TPW>
struct WStage<kW4A16, TPW> {
  uint4 w[TPW];
};
template <int TPW>
struct WStage<kW8A16, TPW> {
  uint4 w[TPW][2];
};

template <int MODE, int MT, int TPW, int NW, int PF>
__global__ __launch_bounds__(64 * NW) void wide_kernel(WideParams p) {
  static_assert(PF >= 2 && PF <= 4, "LDS ring of 2 to 4 slots");
  constexpr int NB = NW * TPW;              // n-tiles per workgroup
  constexpr int XCH = MT * 4;               // 1 KiB activation chunks per group: (m-tile, k-quarter)
  constexpr int XPW = (XCH + NW - 1) / NW;  // chunk loads per wave
  constexpr int XCHP = XPW * NW;            // chunk places per slot (those past XCH: never read)
  constexpr int WLOADS = MODE == kW4A16 ? TPW : 2 * TPW;   // load instructions per weight stage
  // LDS ring: slot r holds the activation chunks of group g (g % PF == r)
  // and each wave's own group scales (W4A16 two fp16 per dword [tile][16];
  // W8A16 one fp16 in the low half of each dword [column]).  One variable per
  // slot, so that reading one slot does not wait for loads into the others.
  // The scales sit after the chunk places, NW * 64 dwords.
  constexpr int SLOT = XCHP * 64 + NW * 16;  // uint4 per slot
  __shared__ __attribute__((aligned(16))) uint4 xs0[SLOT], xs1[SLOT], xs2[SLOT], xs3[SLOT];
  auto xslot = [&](int r) -> uint4* { return r == 0 ? xs0 : r == 1 ? xs1 : r == 2 ? xs2 : xs3; };
  auto sslot = [&](int r) -> uint32_t* { return reinterpret_cast<uint32_t*>(xslot(r) + XCHP * 64); };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, quad = lane >> 4;
  const int nt0 = blockIdx.x * NB;
  const int nvalid = min(NB, p.N / 16 - nt0);
  const int G = p.G;
  const int wt0 = wave * TPW;               // this wave's first n-tile in the workgroup

  const __amdgpu_buffer_rsrc_t rsx = make_rsrc(p.x, (uint32_t)(((int64_t)(p.M - 1) * p.lda + p.K) * 2));
  __amdgpu_buffer_rsrc_t rsw, rss;
  if constexpr (MODE == kW4A16) {
    rsw = make_rsrc(reinterpret_cast<const uint8_t*>(p.w) + (int64_t)nt0 * G * 1024, (uint32_t)(nvalid * G * 1024));
    rss = make_rsrc(p.s + (int64_t)nt0 * G * 16, (uint32_t)(nvalid * G * 32));
  } else {
    rsw = make_rsrc(reinterpret_cast<const int8_t*>(p.w) + (int64_t)nt0 * 16 * p.K, (uint32_t)(nvalid * 16 * (int64_t)p.K));
    rss = make_rsrc(p.s + (int64_t)nt0 * 16 * G, (uint32_t)(nvalid * 16 * G * 2));
  }

  // A slot holds the group's activations as rows of 256 B (128 fp16), row r
  // at r * 256, its 16-byte pieces XOR-swizzled: piece p at position
  // p ^ (r % 16), so that the operand reads below (16 rows, one piece each)
  // hit distinct banks.  LDS-direct load c (c = wave, wave + NW, ...) fills
  // rows 4c .. 4c + 3, one contiguous KiB of each row's group slice: lane l
  // writes position l % 16 of row 4c + l / 16, so it reads piece
  // (l % 16) ^ (row % 16) of that row.  Rows past M read zeros; loads past
  // the tile (c >= XCH) read out of range into places never read, so every
  // wave issues XPW of them and the count of loads per stage is a constant.
  uint32_t vx[XPW];
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int c = wave + NW * i, r = 4 * c + (lane >> 4), piece = (lane & 15) ^ (r & 15);
    vx[i] = c < XCH ? ((uint32_t)r * (uint32_t)p.lda + 8u * piece) * 2u : kOOB;
  }
  // Operand reads: product t of m-tile mt takes, at lane (col, quad), row
  // 16 mt + col, k = 64 (t / 2) + 16 quad + 8 (t % 2) .. + 7 (piece
  // 8 (t / 2) + 2 quad + t % 2), in uint4 units of the slot.
  uint32_t xo[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) xo[t] = (uint32_t)(col * 16 + ((8 * (t >> 1) + 2 * quad + (t & 1)) ^ col));
  // Each wave loads the group scales of its own TPW n-tiles into its 64
  // dwords of the scale slot; lanes past them read out of range (zeros).
  uint32_t vs;
  if constexpr (MODE == kW4A16)   // lane l < 8 TPW: dword l % 8 (scales 2 (l % 8), +1) of tile l / 8
    vs = lane < 8 * TPW ? (((uint32_t)(wt0 + (lane >> 3)) * (uint32_t)G * 16u + 2u * (lane & 7)) * 2u) : kOOB;
  else                            // lane l < 16 TPW: the scale of column l of the wave's tiles
    vs = lane < 16 * TPW ? ((uint32_t)(wt0 * 16 + lane) * (uint32_t)G * 2u) : kOOB;

  // One ring stage: the wave's weights into registers, its chunks and
  // scales into LDS slot r.  Past the last group every load is out of range
  // (reads nothing, writes zeros), so each wave always issues the same
  // number of loads per stage and one constant vmcnt wait covers a stage.
  auto load_w = [&](WStage<MODE, TPW>& st, int g) {
    const uint32_t bad = g < G ? 0u : kOOB;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const uint32_t tj = (uint32_t)(wt0 + j);
      if constexpr (MODE == kW4A16) {
        st.w[j] = ld128_stream(rsw, ((tj * (uint32_t)G + (uint32_t)g) * 64u + lane) * 16u | bad);
      } else {
        const uint32_t row = (tj * 16u + col) * (uint32_t)p.K + (uint32_t)g * 128u + 16u * quad;
        st.w[j][0] = ld128(rsw, row | bad);
        st.w[j][1] = ld128(rsw, (row + 64u) | bad);
      }
    }
  };
  auto load_lds = [&](int g, int r) {
    const uint32_t bad = g < G ? 0u : kOOB;
    uint4* xd = xslot(r);
#pragma unroll
    for (int i = 0; i < XPW; ++i)
      lds16(rsx, &xd[(wave + NW * i) * 64], vx[i] | bad, (uint32_t)g * 256u);
    if constexpr (MODE == kW4A16)
      lds4(rss, &sslot(r)[64 * wave], vs | bad, (uint32_t)g * 32u);
    else
      lds2(rss, &sslot(r)[64 * wave], vs | bad, (uint32_t)g * 2u);
  };
  // Loads a wave issues after group g's LDS loads and before group g is
  // used: the weights of the next PF - 1 groups and the LDS loads of the
  // next PF - 2.
  constexpr int kAfter = (PF - 1) * WLOADS + (PF - 2) * (XPW + 1);

  f32x4 acc[TPW][MT];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x4)0.0f;

  // Prologue: weights of groups 0 .. PF-1, LDS loads of groups 0 .. PF-2,
  // issued group by group.
  WStage<MODE, TPW> st[PF];
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    load_w(st[s], s);
    __builtin_amdgcn_sched_barrier(0);
    if (s < PF - 1) load_lds(s, s);
    __builtin_amdgcn_sched_barrier(0);
  }

  // One group: wait for it, multiply it, refill its ring stage.
  auto step = [&](WStage<MODE, TPW>& stw, const int s, const int g) {
    // Wait for this wave's LDS loads of group g (and so its weights of
    // group g, issued earlier) and its LDS reads of group g - 1, then meet
    // the other waves: after the barrier group g's slot is complete, and
    // every wave is done with group g - 1's slot.  A bare barrier: a
    // release fence would also wait for the LDS loads of later groups.
    static_assert(kAfter < 64, "vmcnt holds 6 bits");
    QG_WAIT_VMCNT_LGKM0(kAfter);
    QG_COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    QG_COMPILER_FENCE();

    const uint4* xr = xslot(s);
    const uint32_t* sr = sslot(s) + 64 * wave;
    f16x8 b[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f16x8 v = __builtin_bit_cast(f16x8, xr[mt * 256 + xo[t]]);
        // W4A16 weight elements come in k order {0,2,4,6,1,3,5,7}; match it.
        if constexpr (MODE == kW4A16)
          b[mt][t] = __builtin_shufflevector(v, v, 0, 2, 4, 6, 1, 3, 5, 7);
        else
          b[mt][t] = v;
      }
    uint2 sv[TPW];   // the lane's 4 fp16 scales per n-tile
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      if constexpr (MODE == kW4A16) {
        sv[j] = *reinterpret_cast<const uint2*>(&sr[j * 8 + 2 * quad]);
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(&sr[j * 16 + 4 * quad]);
        sv[j] = make_uint2(v.x | (v.y << 16), v.z | (v.w << 16));
      }
    }
    // The slot of group g - 1 is free now: refill it with group g + PF - 1.
    // (Scheduling barriers keep each stage's loads in issue order, as the
    // counted wait assumes.)
    __builtin_amdgcn_sched_barrier(0);
    load_lds(g + PF - 1, (s + PF - 1) % PF);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      f16x8 a[4];
      if constexpr (MODE == kW4A16) {
        a[0] = w4_to_f16x8(stw.w[j].x);
        a[1] = w4_to_f16x8(stw.w[j].y);
        a[2] = w4_to_f16x8(stw.w[j].z);
        a[3] = w4_to_f16x8(stw.w[j].w);
      } else {
        a[0] = i8_to_f16x8(stw.w[j][0].x, stw.w[j][0].y);
        a[1] = i8_to_f16x8(stw.w[j][0].z, stw.w[j][0].w);
        a[2] = i8_to_f16x8(stw.w[j][1].x, stw.w[j][1].y);
        a[3] = i8_to_f16x8(stw.w[j][1].z, stw.w[j][1].w);
      }
      const _Float16 sc[4] = {__builtin_bit_cast(_Float16, (uint16_t)(sv[j].x & 0xFFFFu)),
                              __builtin_bit_cast(_Float16, (uint16_t)(sv[j].x >> 16)),
                              __builtin_bit_cast(_Float16, (uint16_t)(sv[j].y & 0xFFFFu)),
                              __builtin_bit_cast(_Float16, (uint16_t)(sv[j].y >> 16))};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[mt][0], (f32x4)0.0f, 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b[mt][1], gs, 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2], b[mt][2], gs, 0, 0, 0);
        gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[3], b[mt][3], gs, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][mt][r] = __builtin_fmaf(gs[r], (float)sc[r], acc[j][mt][r]);
      }
    }
    // refill this stage's registers with group g + PF
    __builtin_amdgcn_sched_barrier(0);
    load_w(stw, g + PF);
    __builtin_amdgcn_sched_barrier(0);
    // The group's products are finished here, before the next group's LDS
    // reads (otherwise two groups' activation operands could be live at once).
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(acc[j][mt]));
  };
  // Whole rings only, with no early exit (the loop's one back edge keeps
  // the compiler's waits exact).  Groups past G read nothing: their weights,
  // activations and scales are out-of-range loads that return zeros, so
  // those steps add exact zeros (acc + 0 * 0 == acc, and acc is never -0).
  for (int g0 = 0; g0 < G; g0 += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) step(st[s], s, g0 + s);
  }

  // No LDS load may still be writing when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(0);

#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    if (wt0 + j >= nvalid) break;
    const int n = (nt0 + wt0 + j) * 16 + 4 * quad;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + col;
      if (m >= p.M) break;
      uint2 o;
      o.x = (uint32_t)float_to_half_bits(acc[j][mt][0]) | ((uint32_t)float_to_half_bits(acc[j][mt][1]) << 16);
      o.y = (uint32_t)float_to_half_bits(acc[j][mt][2]) | ((uint32_t)float_to_half_bits(acc[j][mt][3]) << 16);
      *reinterpret_cast<uint2*>(p.y + (int64_t)m * p.N + n) = o;
    }
  }
}

// Ring depth from the register budget (two waves per SIMD: ~200 VGPRs for
// accumulators, activation operands, converted weights and the ring).
template <int MODE, int MT, int TPW>
constexpr int ring_depth() {
  constexpr int fixed = TPW * MT * 4 + MT * 16 + 16 + 24;
  constexpr int stage = TPW * (MODE == kW4A16 ? 4 : 8);
  constexpr int pf = (200 - fixed) / stage;
  return pf < 2 ? 2 : (pf > 4 ? 4 : pf);
}

// Workgroup shape: NW waves of TPW n-tiles each.  Four tiles per wave
// halve the activation loads and LDS reads per weight byte, but leave room
// for a ring of only two stages; they pay off where the output is wide
// enough to keep 384 such workgroups busy.
struct WideShape {
  int nw, tpw;
};
WideShape wide_shape(int64_t ntiles) {
  if (ntiles >= 32 * 384) return {8, 4};
  if (ntiles >= 16 * 512) return {8, 2};
  if (ntiles >= 8 * 256) return {4, 2};
  return {0, 0};
}

template <int MODE, int MT>
hipError_t launch_mt(const WideParams& p, WideShape sh, hipStream_t st) {
  const int nb = sh.nw * sh.tpw;
  const dim3 grid((unsigned)((p.N / 16 + nb - 1) / nb));
  if (sh.tpw == 4)
    wide_kernel<MODE, MT, 4, 8, ring_depth<MODE, MT, 4>()><<<grid, dim3(64 * 8), 0, st>>>(p);
  else if (sh.nw == 8)
    wide_kernel<MODE, MT, 2, 8, ring_depth<MODE, MT, 2>()><<<grid, dim3(64 * 8), 0, st>>>(p);
  else
    wide_kernel<MODE, MT, 2, 4, ring_depth<MODE, MT, 2>()><<<grid, dim3(64 * 4), 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

int wide_waves(int mode, int64_t M, int64_t N) {
  // Only where the activations are a large share of the traffic (M > 32);
  // at smaller M the K-split kernel streams the weights with more waves per
  // n-tile.
  if ((mode != kW4A16 && mode != kW8A16) || M <= 32 || M > 64) return 0;
  return wide_shape(N / 16).nw;
}

hipError_t launch_wide(const SkinnyArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  WideParams p;
  p.x = reinterpret_cast<const uint16_t*>(a.act);
  p.lda = a.lda;
  p.w = a.w;
  p.s = a.s;
  p.M = (int)a.M;
  p.N = (int)a.N;
  p.K = (int)a.K;
  p.G = (int)(a.K / kGroup);
  p.y = a.y;
  const WideShape sh = wide_shape(a.N / 16);
  if (a.mode == kW4A16)
    return p.M > 48 ? launch_mt<kW4A16, 4>(p, sh, st) : launch_mt<kW4A16, 3>(p, sh, st);
  return p.M > 48 ? launch_mt<kW8A16, 4>(p, sh, st) : launch_mt<kW8A16, 3>(p, sh, st);
}

}  // namespace qg
