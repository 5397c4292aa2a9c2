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
__device__ __forceinline__ f16x8 w4_to_f16x8(uint32_t w) {
  const uint32_t y = w >> 8;
  u32x4 p;
  p[0] = __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64086408u, kBitop3MaskXorElse);
  p[1] = __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64806480u, kBitop3MaskXorElse);
  p[2] = __builtin_amdgcn_bitop3_b32(y, 0x000F000Fu, 0x64086408u, kBitop3MaskXorElse);
  p[3] = __builtin_amdgcn_bitop3_b32(y, 0x00F000F0u, 0x64806480u, kBitop3MaskXorElse);
  const f16x8 v = __builtin_bit_cast(f16x8, p);
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
