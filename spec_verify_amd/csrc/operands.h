// fp16 operands of the fp16 matrix-core products from packed int4 and int8
// weight codes (shared by the weight-streaming kernels).
#pragma once

#include "common.h"

namespace qg {

// Exact fp16 values of the 8 int4 codes of one packed word.  With
// u = nibble ^ 8 = q + 8, the pattern 0x6400 | u is the fp16 number 1024 + u
// and 0x6400 | (u << 4) is 1024 + 16 u; so (v - 1032) and (v / 16 - 72) are
// q exactly.  One shift by 8 serves slots 2, 3, 6, 7.  Element order is
// slots {0, 4, 1, 5, 2, 6, 3, 7} = k offsets {0, 2, 4, 6, 1, 3, 5, 7} (the
// activation operand is shuffled to match).
//
// Each pair of slots is one v_bitop3_b32: out = mask ? (w ^ k) : k, truth
// table 0x6A for operands (w, mask, k), where k holds the exponent pattern
// 0x6400 outside the mask and the nibble's top bit inside it, so the
// sign flip (^ 8), the mask and the exponent insert take one instruction.
constexpr uint32_t kBitop3MaskXorElse = 0x6A;

// The 8 values before the affine step: 1032 + q in elements 0, 1, 4, 5 and
// 1152 + 16 q in elements 2, 3, 6, 7 (all exact in fp16).
__device__ __forceinline__ f16x8 w4_to_f16x8_biased(uint32_t w) {
  const uint32_t y = w >> 8;
  u32x4 p;
  p[0] = __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64086408u, kBitop3MaskXorElse);
  p[1] = __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64806480u, kBitop3MaskXorElse);
  p[2] = __builtin_amdgcn_bitop3_b32(y, 0x000F000Fu, 0x64086408u, kBitop3MaskXorElse);
  p[3] = __builtin_amdgcn_bitop3_b32(y, 0x00F000F0u, 0x64806480u, kBitop3MaskXorElse);
  return __builtin_bit_cast(f16x8, p);
}

// The activation operand that goes with the biased int4 values: elements
// 2, 3, 6, 7 (words 1 and 3) divided by 16, exact for every normal fp16
// quotient.  Then x * (1152 + 16 q) / 16 = 72 x + q x and x * (1032 + q) =
// 1032 x + q x: the contraction is sum(q x) plus a bias that depends on the
// activations alone (w4_bias_operand), which the product takes off by
// starting from minus that bias.
//
// A whole-vector multiply (the compiler drops the factors of 1): taking
// words 1 and 3 out with __builtin_bit_cast(f16x2, u[i]) made the compiler
// read word 0 for both.
__device__ __forceinline__ f16x8 w4_scale_activations(f16x8 x) {
  const f16x8 m = {1.0f16, 1.0f16, 0.0625f16, 0.0625f16, 1.0f16, 1.0f16, 0.0625f16, 0.0625f16};
  return x * m;
}

// A operand whose every row holds the biases with the sign flipped (-1032,
// -1152 in the slots above): its product with the scaled activations is
// minus the bias of each activation column, in all four rows of a lane.
__device__ __forceinline__ f16x8 w4_bias_operand() {
  return f16x8{-1032.0f16, -1032.0f16, -1152.0f16, -1152.0f16, -1032.0f16, -1032.0f16, -1152.0f16, -1152.0f16};
}

__device__ __forceinline__ f16x8 w4_to_f16x8(uint32_t w) {
  const f16x8 v = w4_to_f16x8_biased(w);
  const f16x8 mul = {1.0f16, 1.0f16, 0.0625f16, 0.0625f16, 1.0f16, 1.0f16, 0.0625f16, 0.0625f16};
  const f16x8 add = {-1032.0f16, -1032.0f16, -72.0f16, -72.0f16, -1032.0f16, -1032.0f16, -72.0f16, -72.0f16};
  return v * mul + add;
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

}  // namespace qg
