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
// activations and the group scales of the current 128-wide group are staged
// once per workgroup in LDS (LDS-direct loads: memory to LDS, 16 B per lane
// at consecutive addresses, already in the layout each lane's matrix-core
// operand needs), double buffered with one barrier per group.  So the M x K
// activations pass through a CU once per NW * TPW n-tiles; with K split
// across waves instead (the weight-streaming kernel for narrower outputs)
// every 4 n-tiles re-read them, and at M = 64 that is twice the weight
// bytes.  Weights stream into registers through a PF-deep ring of
// range-checked buffer loads.
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
#define QG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

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
  constexpr int NB = NW * TPW;              // n-tiles per workgroup
  constexpr int XCH = MT * 4;               // 1 KiB activation chunks per group: (m-tile, k-quarter)
  constexpr int WLOADS = MODE == kW4A16 ? TPW : 2 * TPW;   // load instructions per weight stage
  __shared__ __attribute__((aligned(16))) uint4 xs[2][XCH * 64];
  // group scales: W4A16 two fp16 per dword [tile][16]; W8A16 one fp16 in the
  // low half of each dword [column]
  __shared__ __attribute__((aligned(16))) uint32_t ss[2][NB * 16];

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

  // Activation chunk (mt, t) holds, at lane l = col + 16 quad, the 8 fp16 of
  // row 16 mt + col at k = 64 (t / 2) + 16 quad + 8 (t % 2) of the group:
  // exactly the lane's operand of the t-th 16x16x32 product.  Wave w loads
  // chunks w, w + NW, ...; rows past M read zeros.
  constexpr int XPW = (XCH + NW - 1) / NW;  // chunks per wave (the last ones may be past XCH)
  uint32_t vx[XPW];
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int c = min(wave + NW * i, XCH - 1), mt = c >> 2, t = c & 3;
    vx[i] = ((uint32_t)(mt * 16 + col) * (uint32_t)p.lda + 64u * (t >> 1) + 16u * quad + 8u * (t & 1)) * 2u;
  }
  // Scales of the group for the workgroup's 16 * NB columns, as fp16 [column].
  constexpr int SWAVES = MODE == kW4A16 ? (NB * 8 + 63) / 64 : (NB * 16 + 63) / 64;   // waves that load them
  uint32_t vs;
  if constexpr (MODE == kW4A16) {
    const uint32_t d = (uint32_t)(64 * wave + lane);          // dword d: n-tile d / 8, scales 2 (d % 8), +1
    vs = ((d >> 3) * (uint32_t)G * 16u + 2u * (d & 7)) * 2u;
  } else {
    const uint32_t c = (uint32_t)(64 * wave + lane);          // column c of the workgroup
    vs = c * (uint32_t)G * 2u;
  }

  auto lds_load = [&](int g, int buf) {
#pragma unroll
    for (int i = 0; i < XPW; ++i)
      if (wave + NW * i < XCH) lds16(rsx, &xs[buf][(wave + NW * i) * 64], vx[i], (uint32_t)g * 256u);
    if (wave < SWAVES) {
      if constexpr (MODE == kW4A16)
        lds4(rss, &ss[buf][64 * wave], vs, (uint32_t)g * 32u);
      else
        lds2(rss, &ss[buf][64 * wave], vs, (uint32_t)g * 2u);
    }
  };
  auto load_w = [&](WStage<MODE, TPW>& st, int g, bool valid) {
    const uint32_t bad = valid ? 0u : kOOB;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const uint32_t tj = (uint32_t)(wt0 + j);
      if constexpr (MODE == kW4A16) {
        st.w[j] = ld128(rsw, ((tj * (uint32_t)G + (uint32_t)g) * 64u + lane) * 16u + bad);
      } else {
        const uint32_t row = (tj * 16u + col) * (uint32_t)p.K + (uint32_t)g * 128u + 16u * quad;
        st.w[j][0] = ld128(rsw, row + bad);
        st.w[j][1] = ld128(rsw, row + 64u + bad);
      }
    }
  };

  f32x4 acc[TPW][MT];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x4)0.0f;

  WStage<MODE, TPW> st[PF];
#pragma unroll
  for (int s = 0; s < PF; ++s) load_w(st[s], s, s < G);
  lds_load(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int g0 = 0; g0 < G; g0 += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int g = g0 + s;
      if (g >= G) break;                      // uniform across the workgroup
      const int buf = g & 1;
      // This group's activation operands and scales come out of LDS first;
      // then the next group's LDS-direct loads go to the other buffer, so
      // no LDS read here waits behind them.
      f16x8 b[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f16x8 v = __builtin_bit_cast(f16x8, xs[buf][(mt * 4 + t) * 64 + lane]);
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
          sv[j] = *reinterpret_cast<const uint2*>(&ss[buf][(wt0 + j) * 8 + 2 * quad]);
        } else {
          const uint4 v = *reinterpret_cast<const uint4*>(&ss[buf][(wt0 + j) * 16 + 4 * quad]);
          sv[j] = make_uint2(v.x | (v.y << 16), v.z | (v.w << 16));
        }
      }
      if (g + 1 < G) lds_load(g + 1, buf ^ 1);

#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        f16x8 a[4];
        if constexpr (MODE == kW4A16) {
          a[0] = w4_to_f16x8(st[s].w[j].x);
          a[1] = w4_to_f16x8(st[s].w[j].y);
          a[2] = w4_to_f16x8(st[s].w[j].z);
          a[3] = w4_to_f16x8(st[s].w[j].w);
        } else {
          a[0] = i8_to_f16x8(st[s].w[j][0].x, st[s].w[j][0].y);
          a[1] = i8_to_f16x8(st[s].w[j][0].z, st[s].w[j][0].w);
          a[2] = i8_to_f16x8(st[s].w[j][1].x, st[s].w[j][1].y);
          a[3] = i8_to_f16x8(st[s].w[j][1].z, st[s].w[j][1].w);
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
      // refill this stage with group g + PF, then wait for this wave's LDS
      // loads of group g + 1 (issued before the refill, so the refill's loads
      // stay in flight) and meet the other waves
      load_w(st[s], g + PF, g + PF < G);
      QG_WAIT_VMCNT(WLOADS);
      __syncthreads();
    }
  }

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

// Combinations wide_tpw never picks are not instantiated.
template <int MODE, int MT>
hipError_t launch_mt(const WideParams& p, int nw, hipStream_t st) {
  constexpr int TPW = 2;
  const int nb = nw * TPW;
  const dim3 grid((unsigned)((p.N / 16 + nb - 1) / nb));
  if (nw == 8)
    wide_kernel<MODE, MT, TPW, 8, ring_depth<MODE, MT, TPW>()><<<grid, dim3(64 * 8), 0, st>>>(p);
  else
    wide_kernel<MODE, MT, TPW, 4, ring_depth<MODE, MT, TPW>()><<<grid, dim3(64 * 4), 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

int wide_waves(int mode, int64_t M, int64_t N) {
  if ((mode != kW4A16 && mode != kW8A16) || M <= 32 || M > 64) return 0;
  // Only where the activations are a large share of the traffic (M > 32);
  // at smaller M the K-split kernel streams the weights with more waves per
  // n-tile.  Two n-tiles per wave; 8 waves per workgroup (16 n-tiles per
  // activation read) when that still gives 512 workgroups, else 4 when that
  // gives 256.
  const int64_t ntiles = N / 16;
  if (ntiles >= 16 * 512) return 8;
  if (ntiles >= 8 * 256) return 4;
  return 0;
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
  const int nw = wide_waves(a.mode, a.M, a.N);
  if (a.mode == kW4A16)
    return p.M > 48 ? launch_mt<kW4A16, 4>(p, nw, st) : launch_mt<kW4A16, 3>(p, nw, st);
  return p.M > 48 ? launch_mt<kW8A16, 4>(p, nw, st) : launch_mt<kW8A16, 3>(p, nw, st);
}

}  // namespace qg
