// Internal helpers shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kGroup = 128;        // weight / table group width along K
constexpr int kWave = 64;          // CDNA wavefront width

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Kernel launchers (defined next to their kernels).  Shapes are validated by
// the C-ABI layer before any of these is called.
// ---------------------------------------------------------------------------

// Per-token int8 quantisation.  Codes go to q (row-major, leading dimension
// ldq) when q is not null and to qfrag in the fragment order the
// weight-streaming W4A8 kernel reads when qfrag is not null.
hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            int8_t* q, int64_t ldq, int8_t* qfrag, float* scale, hipStream_t st);
// RMSNorm of fp16 rows with an fp16 weight (fp32 math, tree-ordered sum of
// squares), optionally written to y ([M][H]), then quantised exactly as by
// launch_act_quant.  H % 128 == 0, H <= 65536.
hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* w, int64_t M, int64_t H, int64_t ldx, float eps,
                                uint16_t* y, int8_t* q, int64_t ldq, int8_t* qfrag, float* scale, hipStream_t st);

// Split-KV verify attention (head_dim 256): the split plan and the launch of
// both passes.  ws holds ws_bytes (fp32 row maxima, sums and partial rows).
struct AttnPlan {
  int64_t C, S, R;        // positions per split, splits, query rows per KV head
  size_t ml_floats, ws_bytes;
};
AttnPlan attn_plan(int64_t T, int64_t Hq, int64_t Hkv, int64_t L);
hipError_t launch_verify_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int64_t T,
                                   int64_t Hq, int64_t Hkv, int64_t L, void* ws, hipStream_t st);

// Top-k / top-p sampler: chunks of 256*E logits per pass-1 workgroup, C
// chunks per row, kpt candidates per pass-2 thread; E == 0 when the shape is
// beyond the plan (C * k > 16384).
struct SamplerPlan {
  int E;
  int64_t C;
  int kpt;
  size_t ws_bytes;
};
SamplerPlan sampler_plan(int64_t R, int64_t V, int64_t k);
hipError_t launch_sampler(const uint16_t* logits, int64_t R, int64_t V, int64_t ld, int64_t k, float top_p,
                          float temperature, const float* u, int32_t* ids, float* probs, int32_t* kept,
                          int32_t* sampled, float* lse, void* ws, hipStream_t st);

hipError_t launch_w4_repack(const int8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                            void* w_packed, uint16_t* s_packed, hipStream_t st);

// Operating modes of the skinny (M <= 64) GEMM kernel.
enum SkinnyMode { kW4A8 = 0, kW4A16 = 1, kW8A16 = 2 };

// Work decomposition of the skinny kernel: n-tiles (16 columns) per
// workgroup.  A pure function of the operation and shape.
struct SkinnyPlan {
  int nt;       // n-tiles per workgroup: 1, 2 or 4
};
SkinnyPlan skinny_plan(int mode, int64_t N, int64_t K);

struct SkinnyArgs {
  int mode;
  const void* act;          // W4A8: int8 codes in fragment order; W4A16 / W8A16: fp16 [M][lda]
  int64_t lda;
  const float* tok_scale;   // W4A8 token scales [M]
  const void* w;            // packed int4 (W4A8/W4A16) or row-major int8 [N][K] (W8A16)
  const uint16_t* s;        // packed scales (W4A*) or row-major fp16 [N][K/128] (W8A16)
  int64_t M, N, K;
  uint16_t* y;              // fp16 [M][N]
  int32_t* dbg;             // W4A8 debug window (may be null)
  int64_t dm0, dm1, dn0, dn1;
};
hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t st);

// Wide outputs with fp16 activations (W4A16 / W8A16, 32 < M <= 64): waves
// split N and share each group's activations through LDS.  wide_waves gives
// the waves per workgroup the kernel would use for this shape, 0 when the
// weight-streaming kernel runs instead.
int wide_waves(int mode, int64_t M, int64_t N);
hipError_t launch_wide(const SkinnyArgs& a, hipStream_t st);

struct LargeArgs {
  const int8_t* codes;      // [M][K]
  const float* tok_scale;   // [M]
  const void* w;            // packed int4
  const uint16_t* s;        // packed scales
  int64_t M, N, K;
  uint16_t* y;
  int32_t* dbg;
  int64_t dm0, dm1, dn0, dn1;
};
hipError_t launch_w4a8_large(const LargeArgs& a, hipStream_t st);

hipError_t launch_gather(const int32_t* ids, int64_t T, const int8_t* table, const uint16_t* scales,
                         int64_t V, int64_t H, uint16_t* out, hipStream_t st);

hipError_t launch_quant_table(const uint16_t* src, int64_t V, int64_t H, int8_t* Q, uint16_t* S,
                              hipStream_t st);

// Exhaustive check of the quantiser's division: adds the pairs checked to
// counts[0] and the mismatches to counts[1].
hipError_t launch_quant_division_check(unsigned long long* counts, hipStream_t st);
hipError_t launch_probe_read(const void* a, int64_t a_bytes, const void* c, int64_t c_bytes, int share, int wgs,
                             int threads, bool nt, uint32_t* sink, hipStream_t st);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32, round to nearest even
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qg
