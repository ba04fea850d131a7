// Shared pieces of the W4G128 kernels: vector types and the int4 -> fp16
// dequantization used by both the small-batch and the large-batch linear.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace paro {
namespace w4 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Packed codes: one 32-bit word per 8 consecutive channels c0 .. c7, the even
// channels in bits 0..15 and the odd ones in bits 16..31, 4 bits each in
// channel order (word = c0 | c2 << 4 | c4 << 8 | c6 << 12 | c1 << 16 | ...).
// Masking one nibble of each 16-bit half and OR-ing in the fp16 pattern of
// 1024.0 gives the pair (c_{2i}, c_{2i+1}) in channel order: with the mask
// 0x000F000F as 1024 + q, with 0x00F000F0 as 1024 + 16 q. Then (v - (1024 +
// z)) = q - z (or 16 (q - z)) is exact in packed fp16, and one packed multiply
// by s (or s / 16, exact: a power of two) rounds (q - z) s once. Eight values
// cost one shift, four and-or and eight packed fp16 operations.
//
// zz = (1024 + z, 1024 + z), ss = (s, s), zz16 = (1024 + 16 z, ...),
// ss16 = (s / 16, ...); `one` = 0x64006400 held in a vector register, so that
// each (w & mask) | one is a single v_and_or_b32 (the mask is then the only
// scalar operand, as gfx9 encodings allow).
__device__ __forceinline__ h8 dequant8(uint32_t w, h2 zz, h2 ss, h2 zz16, h2 ss16, uint32_t one) {
  const uint32_t w8 = w >> 8;
  const h2 v0 = (__builtin_bit_cast(h2, (w & 0x000F000Fu) | one) - zz) * ss;      // c0, c1
  const h2 v1 = (__builtin_bit_cast(h2, (w & 0x00F000F0u) | one) - zz16) * ss16;  // c2, c3
  const h2 v2 = (__builtin_bit_cast(h2, (w8 & 0x000F000Fu) | one) - zz) * ss;     // c4, c5
  const h2 v3 = (__builtin_bit_cast(h2, (w8 & 0x00F000F0u) | one) - zz16) * ss16; // c6, c7
  h8 out;
  out[0] = v0.x;
  out[1] = v0.y;
  out[2] = v1.x;
  out[3] = v1.y;
  out[4] = v2.x;
  out[5] = v2.y;
  out[6] = v3.x;
  out[7] = v3.y;
  return out;
}

// The fp16 pattern pair of 1024.0 in a vector register (see dequant8).
__device__ __forceinline__ uint32_t fp16_1024_pair() {
  uint32_t v;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(v));
  return v;
}

__device__ __forceinline__ h2 splat2(_Float16 v) { return h2{v, v}; }
__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ uint32_t half_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace w4
}  // namespace paro
