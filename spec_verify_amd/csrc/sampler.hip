// Small-k top-k / top-p sampling of one step's logits.
//
// Source: "What this repo does that stock vLLM doesn't", "In full" item 6.
// With top-k <= 64 known up front, the mask needs only the k largest logits
// of each row, not a sort of the whole 248k-wide row, and the softmax over
// the row is spread over many workgroups instead of one per row.  Target and
// drafts sample from the same truncated support.
//
// Per row r of fp16 logits x (temperature T, top-k k, top-p p, uniform u):
//   ids     the k largest logits, larger first, equal values by lower id
//   mass    softmax of x/T over those k
//   kept    ranks j with sum_{i<j} mass_i < p (rank 0 always)
//   probs   mass renormalised over the kept ranks, 0 after them
//   sampled the id at the smallest kept rank with cumulative probs > u
//   lse     log sum_v exp(x_v / T) over the whole row
//
// Keys.  An element is ranked by the 40-bit key (m(x) << 24) | (2^24-1-id),
// where m maps fp16 bits to an unsigned code in value order (-inf lowest).
// Keys are unique, larger key = earlier rank, and key 0 (m = 0 is a NaN
// pattern, never produced by a real logit) marks padding.
//
// Pass 1: one workgroup of 256 threads per (row, chunk of 256*E logits),
// the chunk held in registers.  Each wave's maximum and sum of
// exp((x - max)/T) go to the workspace (shuffles only), and so do the
// chunk's k largest keys in rank order.  Selection: every wave finds the
// k-th largest of its lanes' own maximum value codes (16 bits) with 16
// ballots, one per bit (at least k keys of the chunk reach it, so all of
// the chunk's top k do); the keys at or above the largest of those
// thresholds, typically a few dozen, are compacted to LDS and ranked by
// counting.  A radix select (8-bit digits, LDS histogram) takes over when
// more than 512 keys survive.
// Pass 2: one workgroup of 512 threads per row selects the k largest of the
// chunks' candidates the same way, combines the waves' partial sums into
// lse, and one wave forms the softmax over the k, the top-p cut (a wave
// prefix sum) and the draw.  All in fp32.
#include "common.h"

namespace qg {
namespace {

constexpr int kMaxK = 64;
constexpr int kP1Threads = 256;
constexpr int kWavesP1 = kP1Threads / 64;   // log-sum-exp partials per chunk
constexpr int kP2Threads = 512;
constexpr uint32_t kIdMask = 0xFFFFFFu;

__device__ __forceinline__ uint32_t unmono16(uint32_t m) { return (m & 0x8000u) ? (m & 0x7FFFu) : (~m & 0xFFFFu); }
__device__ __forceinline__ float h2f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ __forceinline__ uint64_t key_of(uint32_t m, uint32_t id) {
  return ((uint64_t)m << 24) | (uint64_t)(kIdMask - id);
}

constexpr uint32_t kCap = 512;   // survivors ranked directly; more take the radix select

struct SelShared {
  uint32_t hist[256];
  uint32_t bin, above, hb, cnt;
  uint64_t list[kCap];
  uint64_t sorted[kMaxK];
  uint64_t wkey[kP2Threads / 64];
  float wf[kP2Threads / 64];
};

// Sum over the block: wave sums by butterfly, then the waves in order.
template <int NT>
__device__ float block_sum_f32(float v, SelShared& sh) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  if ((threadIdx.x & 63) == 0) sh.wf[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh.wf[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r += sh.wf[i];
  __syncthreads();
  return r;
}

template <int NT>
__device__ float block_max_f32(float v, SelShared& sh) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  if ((threadIdx.x & 63) == 0) sh.wf[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh.wf[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, sh.wf[i]);
  __syncthreads();
  return r;
}

// Radix select over the block: get(j) is this thread's j-th key when it
// takes part (0 otherwise).  Returns the largest thr such that at least
// `need` taking keys are >= thr; when those keys are distinct, exactly
// `need` of them are.  The caller guarantees at least `need` taking keys.
// Digits are 8 bits from the top of the 40-bit key; the search stops early
// once the bucket holding the need-th key is taken whole.
template <int NT, int KPT, typename Get>
__device__ uint64_t block_kth(Get get, uint32_t need, SelShared& sh) {
  uint64_t prefix = 0;
  int sft = 32;
  for (int d = 4; d >= 0; --d) {
    sft = 8 * d;
    for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t q = get(j);
      if (q != 0 && (q >> (sft + 8)) == prefix) atomicAdd(&sh.hist[(uint32_t)(q >> sft) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // Lane l owns bins 4l .. 4l+3; the keys above them sit in lanes > l.
      const int l = threadIdx.x;
      uint32_t hs[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) hs[b] = sh.hist[4 * l + b];
      const uint32_t c = hs[0] + hs[1] + hs[2] + hs[3];
      uint32_t incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = (uint32_t)__shfl_down((int)incl, o);
        if (l + o < 64) incl += t;
      }
      uint32_t above = incl - c;
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (above < need && above + hs[b] >= need) {
          sh.bin = (uint32_t)(4 * l + b);
          sh.above = above;
          sh.hb = hs[b];
        }
        above += hs[b];
      }
    }
    __syncthreads();
    const uint32_t bin = sh.bin, above = sh.above, hb = sh.hb;
    __syncthreads();
    need -= above;
    prefix = (prefix << 8) | bin;
    if (hb == need) break;
  }
  return prefix << sft;
}

// Moves the keys >= thr (distinct, at most kMaxK of them) to sh.list in no
// particular order; returns how many there are.
template <int NT, int KPT, typename Get>
__device__ uint32_t block_collect(Get get, uint64_t thr, SelShared& sh) {
  if (threadIdx.x == 0) sh.cnt = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint64_t q = get(j);
    if (q != 0 && q >= thr) {
      const uint32_t slot = atomicAdd(&sh.cnt, 1u);
      if (slot < (uint32_t)kMaxK) sh.list[slot] = q;
    }
  }
  __syncthreads();
  const uint32_t n = sh.cnt;
  __syncthreads();
  return n < (uint32_t)kMaxK ? n : (uint32_t)kMaxK;
}

// The k-th largest of the wave's 64 16-bit values (0 when fewer than k are
// nonzero): the largest t with at least k lanes >= t, built bit by bit with
// ballots.  No LDS, no barrier.
__device__ __forceinline__ uint32_t wave_kth16(uint32_t m, uint32_t k) {
  uint32_t t = 0;
#pragma unroll
  for (int b = 15; b >= 0; --b) {
    const uint32_t tr = t | (1u << b);
    if ((uint32_t)__popcll(__ballot(m >= tr)) >= k) t = tr;
  }
  return t;
}

// The block's k largest keys, sorted (larger first) into sh.sorted[0..k),
// zeros after the last when the block holds fewer than k.  get(j, tau)
// returns this thread's j-th key when it is nonzero and >= tau, else 0;
// tmaxm is the value code (key >> 24) of this thread's largest key.
//
// Threshold: in each wave, the k-th largest of the lanes' value codes is a
// lower bound of the block's k-th largest value (k keys reach it), and so
// is the largest of them over the waves; tau is that value with the id bits
// zero.  The keys >= tau (typically a few dozen) are compacted to LDS, one
// atomic per wave and step, and ranked by counting; past kCap survivors the
// radix select takes over.
template <int NT, int KPT, typename Get>
__device__ void block_topk(Get get, uint32_t tmaxm, uint32_t k, SelShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t tw = wave_kth16(tmaxm, k);
  if (lane == 0) sh.wkey[tid >> 6] = tw;
  if (tid == 0) sh.cnt = 0;
  for (int i = tid; i < (int)k; i += NT) sh.sorted[i] = 0;
  __syncthreads();
  uint64_t tau = sh.wkey[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) tau = sh.wkey[i] > tau ? sh.wkey[i] : tau;
  tau <<= 24;
  if (__ballot(tmaxm >= (uint32_t)(tau >> 24) && tmaxm != 0)) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t q = get(j, tau);
      const uint64_t mask = __ballot(q != 0);
      if (mask) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&sh.cnt, (uint32_t)__popcll(mask));
        base = (uint32_t)__shfl((int)base, 0);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (q != 0 && base + below < kCap) sh.list[base + below] = q;
      }
    }
  }
  __syncthreads();
  const uint32_t n = sh.cnt;
  if (n <= kCap) {
    // Zero keys pad the list to a multiple of 8 (they rank below every
    // key), so the count below reads 16-byte pairs, four at a time.
    const uint32_t n8 = (n + 7) & ~7u;
    if ((uint32_t)tid < n8 - n) sh.list[n + tid] = 0;
    __syncthreads();
    const uint4* l2 = reinterpret_cast<const uint4*>(sh.list);
    for (int i = tid; i < (int)n; i += NT) {
      const uint64_t mine = sh.list[i];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < n8 / 2; j += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 pr = l2[j + u];
          rank += (((uint64_t)pr.y << 32) | pr.x) > mine ? 1u : 0u;
          rank += (((uint64_t)pr.w << 32) | pr.z) > mine ? 1u : 0u;
        }
      }
      if (rank < k) sh.sorted[rank] = mine;
    }
  } else {
    __syncthreads();
    auto g2 = [&](int j) { return get(j, tau); };
    const uint64_t thr = block_kth<NT, KPT>(g2, k, sh);
    block_collect<NT, KPT>(g2, thr, sh);
    if ((uint32_t)tid < k) {
      const uint64_t mine = sh.list[tid];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < k; ++j) rank += sh.list[j] > mine ? 1u : 0u;
      if (rank < k) sh.sorted[rank] = mine;
    }
  }
  __syncthreads();
}

struct ChunkArgs {
  const uint16_t* x;
  int64_t ld;
  int V, C, k;
  float c1;              // log2(e) / T
  uint64_t* wkeys;       // [R][C][k]
  float2* wstat;         // [R][C][kWavesP1]: each wave's maximum of x, sum of exp2((x - max) * c1)
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Value codes of two packed fp16 values: h ^ 0x8000 for a positive value,
// h ^ 0xFFFF for a negative one.
__device__ __forceinline__ uint32_t mono16x2(uint32_t w) {
  const uint32_t neg = (w >> 15) & 0x00010001u;
  return w ^ (0x80008000u | (neg * 0x7FFFu));
}

template <int E>
__global__ __launch_bounds__(kP1Threads) void sampler_chunk_kernel(ChunkArgs a) {
  constexpr int NT = kP1Threads, NV = E / 8, CH = NT * E;
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int c = (int)(blockIdx.x % (unsigned)a.C);
  const int r = (int)(blockIdx.x / (unsigned)a.C);
  const uint16_t* row = a.x + (int64_t)r * a.ld;
  const int c0 = c * CH;

  // Load: vector i of this thread holds elements c0 + 8 (tid + NT i) + 0..7,
  // as packed fp16 pairs w and their packed value codes mp.  Past V (the
  // last chunk only) a value reads as -inf, which adds nothing to the sum,
  // and its code is 0, which is never selected.
  uint32_t w[E / 2], mp[E / 2];
  if (c0 + CH <= a.V) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      // logits are read once: non-temporal hint
      const uint4 v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(row + c0 + 8 * (tid + NT * i))));
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < E / 2; ++i) mp[i] = mono16x2(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int g = c0 + 8 * (tid + NT * i);
      uint32_t h[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) h[t] = g + t < a.V ? (uint32_t)row[g + t] : 0xFC00u;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w[4 * i + t] = h[2 * t] | (h[2 * t + 1] << 16);
        const uint32_t m = mono16x2(w[4 * i + t]);
        mp[4 * i + t] = (g + 2 * t < a.V ? m & 0xFFFFu : 0u) | (g + 2 * t + 1 < a.V ? m & 0xFFFF0000u : 0u);
      }
    }
  }
  auto gid = [&](int e) { return (uint32_t)(c0 + 8 * (tid + NT * (e >> 3)) + (e & 7)); };
  auto code = [&](int e) { return (mp[e >> 1] >> (16 * (e & 1))) & 0xFFFFu; };

  // The thread's largest value code (packed maximum, then the two halves).
  u16x2 pm = __builtin_bit_cast(u16x2, mp[0]);
#pragma unroll
  for (int i = 1; i < E / 2; ++i) pm = __builtin_elementwise_max(pm, __builtin_bit_cast(u16x2, mp[i]));
  const uint32_t tmaxm = pm.x > pm.y ? pm.x : pm.y;

  // The wave's maximum and sum of exponentials (the full softmax's
  // partials, one pair per wave: shuffles only, no barrier).
  uint32_t wmaxm = tmaxm;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) wmaxm = max(wmaxm, (uint32_t)__shfl_xor((int)wmaxm, m));
  // (A wave past the end of the row holds no logit: code 0, maximum -inf.)
  const float xmax = wmaxm ? h2f(unmono16(wmaxm)) : -INFINITY;
  float s = 0.0f;
  if (xmax != -INFINITY) {
    const float off = xmax * a.c1;
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      const f16x2 hv = __builtin_bit_cast(f16x2, w[i]);
      s += __builtin_amdgcn_exp2f(__builtin_fmaf((float)hv.x, a.c1, -off));
      s += __builtin_amdgcn_exp2f(__builtin_fmaf((float)hv.y, a.c1, -off));
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if ((tid & 63) == 0) a.wstat[((int64_t)r * a.C + c) * kWavesP1 + (tid >> 6)] = make_float2(xmax, s);

  // The chunk's k largest keys, in rank order.
  const uint32_t k = (uint32_t)a.k;
  auto getk = [&](int e, uint64_t tau) -> uint64_t {
    const uint32_t m = code(e);
    if (m == 0 || m < (uint32_t)(tau >> 24)) return 0;
    return key_of(m, gid(e));
  };
  block_topk<NT, E>(getk, tmaxm, k, sh);
  uint64_t* out = a.wkeys + ((int64_t)r * a.C + c) * a.k;
  if ((uint32_t)tid < k) out[tid] = sh.sorted[tid];
}

struct RowArgs {
  const uint64_t* wkeys;
  const float2* wstat;
  int C, k;
  float c1, T, top_p;
  const float* u;
  int32_t* ids;
  float* probs;
  int32_t* kept;
  int32_t* sampled;
  float* lse;
};

template <int KPT>
__global__ __launch_bounds__(kP2Threads) void sampler_row_kernel(RowArgs a) {
  constexpr int NT = kP2Threads;
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int nk = a.C * a.k;
  const uint64_t* keys = a.wkeys + (int64_t)r * nk;
  const int nst = a.C * kWavesP1;
  const float2* stat = a.wstat + (int64_t)r * nst;
  // The first NT of the chunks' partial sums load with the candidates.
  const float2 st0 = tid < nst ? stat[tid] : make_float2(-INFINITY, 0.0f);
  uint64_t q[KPT];
  uint64_t tmax = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + NT * j;
    q[j] = i < nk ? keys[i] : 0;
    tmax = q[j] > tmax ? q[j] : tmax;
  }
  const uint32_t k = (uint32_t)a.k;

  auto getk = [&](int j, uint64_t tau) -> uint64_t { return q[j] >= tau ? q[j] : 0; };
  block_topk<NT, KPT>(getk, (uint32_t)(tmax >> 24), k, sh);

  // Full-row log-sum-exp from the chunks' maxima and sums.
  float xm = st0.x;
  for (int c = tid + NT; c < nst; c += NT) xm = fmaxf(xm, stat[c].x);
  const float X = block_max_f32<NT>(xm, sh);
  float part = st0.x != -INFINITY ? st0.y * exp2f((st0.x - X) * a.c1) : 0.0f;
  for (int c = tid + NT; c < nst; c += NT) {
    const float2 st = stat[c];
    if (st.x != -INFINITY) part += st.y * exp2f((st.x - X) * a.c1);
  }
  const float S = block_sum_f32<NT>(part, sh);

  if (tid < 64) {
    const int j = tid;
    const bool in = (uint32_t)j < k;
    const uint64_t key = in ? sh.sorted[j] : 0;
    const float x = in ? h2f(unmono16((uint32_t)(key >> 24))) : 0.0f;
    const int id = in ? (int)(kIdMask - (uint32_t)(key & kIdMask)) : 0;
    const float x0 = __shfl(x, 0);
    const float e = in ? exp2f((x - x0) * a.c1) : 0.0f;
    float cum = e;                                   // inclusive prefix sum over the ranks
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(cum, o);
      if (j >= o) cum += t;
    }
    const float total = __shfl(cum, 63);
    float before = __shfl_up(cum, 1);
    if (j == 0) before = 0.0f;
    const uint64_t kb = __ballot(in && before < a.top_p * total);
    const int nkept = __popcll(kb);                  // a prefix of the ranks; rank 0 always
    const float ks = __shfl(cum, nkept - 1);
    const float uu = a.u[r];
    const uint64_t sb = __ballot(j < nkept && cum <= uu * ks);
    const int rank = min(__popcll(sb), nkept - 1);
    const int sid = __shfl(id, rank);
    if (in) {
      a.ids[(int64_t)r * a.k + j] = id;
      a.probs[(int64_t)r * a.k + j] = j < nkept ? e / ks : 0.0f;
    }
    if (j == 0) {
      a.kept[r] = nkept;
      a.sampled[r] = sid;
      a.lse[r] = X / a.T + logf(S);
    }
  }
}

int chunk_elems(int64_t R, int64_t V, int64_t k) {
  // Chunks of 4096 logits where that still gives two workgroups per CU
  // (>= 512), else 2048, within pass 2's candidate capacity (C * k <= 512
  // threads x 32); otherwise the smallest chunk that fits.  Over 248,320
  // logits: 16 rows took 15.7 us with 4096 against 16.7 us with 2048; one
  // row took 13.4 us against 12.9 us, so it keeps 2048.
  for (int E : {16, 8}) {
    const int64_t C = (V + 256 * E - 1) / (256 * E);
    if (R * C >= 512 && C * k <= (int64_t)kP2Threads * 32) return E;
  }
  for (int E : {8, 16, 32}) {
    const int64_t C = (V + 256 * E - 1) / (256 * E);
    if (C * k <= (int64_t)kP2Threads * 32) return E;
  }
  return 0;
}

}  // namespace

SamplerPlan sampler_plan(int64_t R, int64_t V, int64_t k) {
  SamplerPlan pl{};
  pl.E = chunk_elems(R, V, k);
  if (pl.E == 0) return pl;
  pl.C = (V + 256 * pl.E - 1) / (256 * pl.E);
  const int64_t per = (pl.C * k + kP2Threads - 1) / kP2Threads;
  pl.kpt = 1;
  while (pl.kpt < per) pl.kpt *= 2;
  pl.ws_bytes = (size_t)(R * pl.C * k) * 8 + (size_t)(R * pl.C * kWavesP1) * 8;
  return pl;
}

hipError_t launch_sampler(const uint16_t* logits, int64_t R, int64_t V, int64_t ld, int64_t k, float top_p,
                          float temperature, const float* u, int32_t* ids, float* probs, int32_t* kept,
                          int32_t* sampled, float* lse, void* ws, hipStream_t st) {
  const SamplerPlan pl = sampler_plan(R, V, k);
  ChunkArgs ca;
  ca.x = logits;
  ca.ld = ld;
  ca.V = (int)V;
  ca.C = (int)pl.C;
  ca.k = (int)k;
  ca.c1 = 1.4426950408889634f / temperature;
  ca.wkeys = reinterpret_cast<uint64_t*>(ws);
  ca.wstat = reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) + (size_t)(R * pl.C * k) * 8);
  const dim3 g1((unsigned)(R * pl.C));
  switch (pl.E) {
    case 32: sampler_chunk_kernel<32><<<g1, kP1Threads, 0, st>>>(ca); break;
    case 16: sampler_chunk_kernel<16><<<g1, kP1Threads, 0, st>>>(ca); break;
    default: sampler_chunk_kernel<8><<<g1, kP1Threads, 0, st>>>(ca); break;
  }
  RowArgs ra;
  ra.wkeys = ca.wkeys;
  ra.wstat = ca.wstat;
  ra.C = (int)pl.C;
  ra.k = (int)k;
  ra.c1 = ca.c1;
  ra.T = temperature;
  ra.top_p = top_p;
  ra.u = u;
  ra.ids = ids;
  ra.probs = probs;
  ra.kept = kept;
  ra.sampled = sampled;
  ra.lse = lse;
  const dim3 g2((unsigned)R);
  switch (pl.kpt) {
    case 1: sampler_row_kernel<1><<<g2, kP2Threads, 0, st>>>(ra); break;
    case 2: sampler_row_kernel<2><<<g2, kP2Threads, 0, st>>>(ra); break;
    case 4: sampler_row_kernel<4><<<g2, kP2Threads, 0, st>>>(ra); break;
    case 8: sampler_row_kernel<8><<<g2, kP2Threads, 0, st>>>(ra); break;
    case 16: sampler_row_kernel<16><<<g2, kP2Threads, 0, st>>>(ra); break;
    default: sampler_row_kernel<32><<<g2, kP2Threads, 0, st>>>(ra); break;
  }
  return hipGetLastError();
}

}  // namespace qg
