// MFMA operand helpers shared by the linear kernels and the persistent decode
// kernel: which k-slots a lane feeds to each v_mfma_f32_16x16x32_bf16 of a
// 128-wide chunk, and the exact conversion of int8 / 4-bit codes to bf16.
#pragma once

#include "common.h"
#include "kernels.h"

namespace er {

// LDS/register column (in bf16 elements within the 128-wide chunk) of the 8
// k-slots that lane group kb feeds to MFMA number i; the same mapping decides
// which weight bytes a lane loads, so A and B agree on every k.
template <int FMT>
ER_DEV int kcol(int i, int kb) {
  if constexpr (FMT == FMT_BF16) return 32 * i + 8 * kb;
  else if constexpr (FMT == FMT_W8) return 64 * (i >> 1) + 16 * kb + 8 * (i & 1);
  else return 32 * kb + 8 * i;
}

// Kernel layout of a W4 matrix [N][K]: rows in groups of 8; within a group,
// the 64-byte pieces of 128 codes are stored chunk after chunk, the group's
// rows adjacent within a chunk.  Byte offset of the piece of row n, chunk c
// (the last group may hold fewer than 8 rows; the matrix stays N * K / 2
// bytes).  A 16-row tile made of two aligned 8-row groups (consecutive rows,
// or the paired halves the fused epilogues use) reads two 512-byte runs per
// chunk instead of 16 pieces one row stride apart.
ER_DEV long w4_piece(long n, long c, long N, long K) {
  const long g8 = n & ~7L;
  const long rows = N - g8 < 8 ? N - g8 : 8;
  return g8 * (K >> 1) + c * rows * 64 + (n & 7) * 64;
}

// 8 int8 codes (two words) -> bf16 of (q + 128), exact.
ER_DEV bf16x8_t w8_to_bf16(uint32_t a, uint32_t b) {
  a ^= 0x80808080u;
  b ^= 0x80808080u;
  uint32_t r[4];
  const uint32_t src[2] = {a, b};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float f0 = (float)(src[h] & 0xFFu), f1 = (float)((src[h] >> 8) & 0xFFu);
    const float f2 = (float)((src[h] >> 16) & 0xFFu), f3 = (float)(src[h] >> 24);
    r[2 * h] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
    r[2 * h + 1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
  }
  return __builtin_bit_cast(bf16x8_t, *(const uint4*)r);
}

// One kernel-order W4 word (8 codes) -> bf16 of (q + 128), exact: the code
// lands in the mantissa of 128.0.
ER_DEV bf16x8_t w4_to_bf16(uint32_t w) {
  // (w >> 4j) & 0x000F000F | 0x43004300.  The two constants come from
  // opaque moves (mask in an SGPR, magic in a VGPR) so that the compiler
  // selects one v_and_or_b32 per word instead of an and + an or with literal
  // operands; the arithmetic itself stays plain code.
  uint32_t mask, magic;
  asm("s_mov_b32 %0, 0x000F000F" : "=s"(mask));
  asm("v_mov_b32 %0, 0x43004300" : "=v"(magic));
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = ((w >> (4 * j)) & mask) | magic;
  return __builtin_bit_cast(bf16x8_t, *(const uint4*)r);
}

}  // namespace er
